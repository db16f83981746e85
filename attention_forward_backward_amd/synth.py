"""Seeded synthetic inputs for attention: Q, K, V and the output gradient dO.

This module holds no attention arithmetic. It is the one piece shared by the
HIP path's callers (tests, bench) and by the oracle's callers: both sides are
handed the same arrays, and neither imports the other.

Generator (counter-based, every element addressable by its index):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the output for counter value ``c`` is
  ``mix64(c)`` with the published finaliser (xor-shift 30, multiply by
  0xBF58476D1CE4E5B9, xor-shift 27, multiply by 0x94D049BB133111EB,
  xor-shift 31), and the sequential generator advances its state by the
  golden-ratio increment 0x9E3779B97F4A7C15 before each output.
* Stream key for (seed, tensor id): ``kappa = mix64(((seed << 8) | tid) + G)``
  with ``G`` the increment above.  Tensor ids: Q = 0, K = 1, V = 2, dO = 3.
* Element ``i`` of the flat row-major [B, H, S, D] tensor takes two words
  ``a = mix64(kappa + (2i + 1) G)`` and ``b = mix64(kappa + (2i + 2) G)``
  (all arithmetic mod 2**64), which become uniforms
  ``u1 = ((a >> 11) + 1) / 2**53`` in (0, 1] and ``u2 = (b >> 11) / 2**53``
  in [0, 1).
* Box-Muller, cosine branch: ``z = sqrt(-2 ln u1) cos(2 pi u2)`` in float64,
  times sigma, rounded to float32 (round to nearest even).
* The bf16 variant rounds that float32 value to bfloat16, round to nearest
  even, so a bf16 input is exactly representable in float32 and float64.

Workload shapes follow the five attention configurations this library is
measured on (tiny, small decoder, decoder training step, long context,
ragged encoder); see ``CONFIGS``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on one Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def splitmix64_sequence(state: int, n: int) -> list[int]:
    """The sequential SplitMix64 generator: add G, then mix, n times."""
    out = []
    for _ in range(n):
        state = (state + GOLDEN) & MASK64
        out.append(mix64_int(state))
    return out


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= np.uint64(_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(_M2)
    z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, tensor_id: int) -> int:
    if not (0 <= seed < (1 << 55)) or not (0 <= tensor_id < 256):
        raise ValueError("seed must be in [0, 2**55) and tensor_id in [0, 256)")
    return mix64_int(((seed << 8) | tensor_id) + GOLDEN)


def uniforms(seed: int, tensor_id: int, start: int, count: int):
    """(u1, u2) float64 arrays for flat element indices start .. start+count-1."""
    kappa = np.uint64(stream_key(seed, tensor_id))
    g = np.uint64(GOLDEN)
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        a = _mix64(kappa + (np.uint64(2) * idx + np.uint64(1)) * g)
        b = _mix64(kappa + (np.uint64(2) * idx + np.uint64(2)) * g)
    scale53 = 2.0 ** -53
    u1 = ((a >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * scale53
    u2 = (b >> np.uint64(11)).astype(np.float64) * scale53
    return u1, u2


def normal_f32(seed: int, tensor_id: int, shape, sigma: float = 1.0,
               start: int = 0) -> np.ndarray:
    """float32 array of N(0, sigma^2) samples, row-major over ``shape``."""
    n = int(np.prod(shape)) if len(shape) else 1
    u1, u2 = uniforms(seed, tensor_id, start, n)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return (sigma * z).astype(np.float32).reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16, nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding here is defined for finite inputs only")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class AttnConfig:
    name: str
    batch: int
    heads: int
    seq: int
    head_dim: int
    causal: bool
    sigma_qkv: float
    sigma_do: float
    dtypes: tuple

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def shape(self):
        return (self.batch, self.heads, self.seq, self.head_dim)

    @property
    def pairs(self) -> int:
        """Visible (query, key) pairs: S(S+1)/2 per head if causal, else S^2."""
        s = self.seq
        per = s * (s + 1) // 2 if self.causal else s * s
        return self.batch * self.heads * per

    @property
    def flops(self) -> dict:
        """Credited FLOP: forward 4*D per pair (QK^T, PV), backward 10*D per
        pair (QK^T recompute, dO V^T, P^T dO, dS K, dS^T Q)."""
        d = self.head_dim
        return {"fwd": 4 * d * self.pairs, "bwd": 10 * d * self.pairs,
                "fwd_bwd": 14 * d * self.pairs}


# The five measured workloads (sizes, causal flag, input distributions).
CONFIGS = {
    "tiny": AttnConfig("tiny", 1, 2, 64, 32, True, 1.0, 1.0, ("f32",)),
    "small_decoder": AttnConfig("small_decoder", 4, 8, 256, 64, True, 1.0, 1.0, ("f32",)),
    "decoder_step": AttnConfig("decoder_step", 8, 12, 512, 64, True, 1.0, 1.0, ("f32", "bf16")),
    "long_context": AttnConfig("long_context", 1, 16, 1024, 128, True, 1.0, 1.0, ("f32", "bf16")),
    "ragged_encoder": AttnConfig("ragged_encoder", 32, 8, 197, 64, False, 0.5, 1.0, ("f32", "bf16")),
}


def make_inputs(shape, seed: int, dtype: str = "f32", sigma_qkv: float = 1.0,
                sigma_do: float = 1.0) -> dict:
    """Q, K, V, dO for one run.

    Returns a dict of float32 arrays holding the exact values the GPU sees
    (for ``dtype == "bf16"`` they are the bf16-rounded values, widened), and,
    for bf16, the raw uint16 bit arrays under ``"<name>_bits"``.
    """
    out = {}
    for name, tid in TENSOR_IDS.items():
        sigma = sigma_do if name == "do" else sigma_qkv
        x = normal_f32(seed, tid, shape, sigma)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_bits"] = bits
            x = bf16_bits_to_f32(bits)
        elif dtype != "f32":
            raise ValueError(f"unknown dtype {dtype!r}")
        out[name] = x
    return out


def config_inputs(cfg: AttnConfig, seed: int, dtype: str) -> dict:
    return make_inputs(cfg.shape, seed, dtype, cfg.sigma_qkv, cfg.sigma_do)


@dataclass(frozen=True)
class CrossWorkload:
    """A query/key-length pair with optional per-batch valid key counts."""
    name: str
    batch: int
    heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    causal: bool
    padded: bool  # per-batch valid key counts drawn by ``key_lengths``
    min_keys: int = 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# Cross-attention and one-token workloads: a 77-token text-conditioning
# cross-attention over a 64x64 latent grid (4096 queries), and a one-token
# query over a 512-key context, with all keys valid or with padded batches.
CROSS_WORKLOADS = {
    "text_cross": CrossWorkload("text_cross", 2, 8, 4096, 77, 64, False, False),
    "decode": CrossWorkload("decode", 8, 12, 1, 512, 64, True, False),
    "decode_padded": CrossWorkload("decode_padded", 8, 12, 1, 512, 64, True, True, 64),
}

KEY_LENGTH_TENSOR_ID = 16


def key_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """int32 [batch] of valid key counts, uniform on lo..hi inclusive, from the
    u2 uniforms of the generator's stream KEY_LENGTH_TENSOR_ID."""
    if not 0 <= lo <= hi:
        raise ValueError("need 0 <= lo <= hi")
    _, u2 = uniforms(seed, KEY_LENGTH_TENSOR_ID, 0, batch)
    return (lo + np.floor(u2 * (hi - lo + 1))).astype(np.int32)


def cross_inputs(shape_q, shape_k, seed: int, dtype: str = "f32") -> dict:
    """Q and dO of shape ``shape_q``, K and V of shape ``shape_k`` (the keys
    come from seed + 100, so they differ from a same-seed query draw)."""
    qi = make_inputs(shape_q, seed, dtype)
    ki = make_inputs(shape_k, seed + 100, dtype)
    out = {n: qi[n] for n in ("q", "do")}
    out.update({n: ki[n] for n in ("k", "v")})
    if dtype == "bf16":
        out.update({n + "_bits": qi[n + "_bits"] for n in ("q", "do")})
        out.update({n + "_bits": ki[n + "_bits"] for n in ("k", "v")})
    return out


# Convolution inputs: x [N,H,W,C], w [K,R,S,C] and dy [N,P,Q,K] from streams
# of their own.
CONV_TENSOR_IDS = {"x": 20, "w": 21, "dy": 22}


def conv_inputs(x_shape, w_shape, dy_shape, seed: int, dtype: str = "f32") -> dict:
    """x, w, dy ~ N(0, 1) as float32 arrays holding the exact values the GPU
    sees (bf16-rounded for ``dtype == "bf16"``, with the raw bits under
    "<name>_bits"); w is drawn with sigma 1/sqrt(R*S*C), so that y is of
    unit size."""
    K, R, S, C = w_shape
    out = {}
    for name, shape in (("x", x_shape), ("w", w_shape), ("dy", dy_shape)):
        sigma = 1.0 / math.sqrt(R * S * C) if name == "w" else 1.0
        x = normal_f32(seed, CONV_TENSOR_IDS[name], shape, sigma)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_bits"] = bits
            x = bf16_bits_to_f32(bits)
        elif dtype != "f32":
            raise ValueError(f"unknown dtype {dtype!r}")
        out[name] = x
    return out


# Longer causal self-attention shapes the benchmark times beside the five
# workloads: the decoder-step token count at S = 2048 and 4096, and a long
# head_dim-128 set, (B, H, S, D).
LONG_SEQ_SHAPES = [(2, 12, 2048, 64), (1, 12, 4096, 64), (1, 16, 4096, 128)]

# ResNet-50 convolutions at batch 32 and 224 x 224 input (the pages' ResNet-50
# workload; its batch and image size are not given): name -> (N, H, W, C, K,
# R, S, stride, pad).  The stem's input is the image, which takes no
# gradient, so it has no data derivative.
CONV_LAYERS = {
    "stem_7x7_s2": (32, 224, 224, 3, 64, 7, 7, (2, 2), (3, 3)),
    "conv2_3x3": (32, 56, 56, 64, 64, 3, 3, (1, 1), (1, 1)),
    "conv4_1x1": (32, 14, 14, 1024, 256, 1, 1, (1, 1), (0, 0)),
}
