"""MI355X (gfx950) fused attention forward/backward: Python binding.

A thin ctypes layer over ``libattn_mi355x.so`` (the C ABI in
``include/attn.h``).  The functions here have the C names and only marshal
arguments: torch tensors supply device pointers and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = ["AttnError", "lib", "attn_fwd", "attn_fwd_ws", "attn_fwd_workspace_size", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_prep",
           "attn_bwd_dkdv",
           "attn_bwd_dq", "attn_bwd_workspace_size", "attn_bwd_workspace_size_min",
           "attn_fwd_cross", "attn_bwd_cross", "attn_bwd_cross_workspace_size",
           "attn_bwd_cross_workspace_size_min",
           "attn_fwd_rope", "attn_bwd_rope",
           "attn_status_string", "attn_version", "conv2d_fwd", "conv2d_bwd_data",
           "conv2d_bwd_filter", "conv2d_bwd_filter_workspace_size", "conv2d_out_size",
           "ATTN_F32", "ATTN_BF16", "ATTN_F32_BF16FWD", "STATUS", "LIB_PATH", "HEADER_PATH"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "attn.h")
CONV_HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "conv.h")

ATTN_F32, ATTN_BF16, ATTN_F32_BF16FWD = 0, 1, 2
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
          3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}


class AttnError(RuntimeError):
    def __init__(self, func: str, code: int):
        self.code = code
        super().__init__(f"{func} returned {STATUS.get(code, code)}")


_lib = None
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "attn_fwd": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_cross": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _F, _P]),
    "attn_fwd_ws": (_I, [_I, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_bwd_cross": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                            _I, _I, _I, _I, _I, _P, _I, _F, _P]),
    "attn_bwd_cross_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_bwd_cross_workspace_size_min": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_bwd_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_bwd_workspace_size_min": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_bwd_prep": (_I, [_I, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _P]),
    "attn_bwd": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                      _I, _I, _I, _I, _I, _F, _P]),
    "attn_bwd_noalloc": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _I, _I, _I, _I, _I, _F, _P]),
    "attn_bwd_dq": (_I, [_I, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _P]),
    "attn_bwd_dkdv": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_strided": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P,
                              ctypes.POINTER(ctypes.c_longlong), _I, _F, _P]),
    "attn_bwd_strided": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I,
                              _I, _P, ctypes.POINTER(ctypes.c_longlong), _I, _F, _P]),
    "attn_fwd_rope": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                           ctypes.POINTER(ctypes.c_longlong), _P, _P, _I, _I, _I, _F, _P]),
    "attn_bwd_rope": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I,
                           ctypes.POINTER(ctypes.c_longlong), _P, _P, _I, _I, _I, _F, _P]),
    "attn_rope_copy": (_I, [_I, _P, ctypes.POINTER(ctypes.c_longlong), _P,
                            ctypes.POINTER(ctypes.c_longlong), _P, _P, _I, _I, _I, _I, _I, _I,
                            _I, _P]),
    "conv2d_fwd": (_I, [_I, _P, _P, _P] + [_I] * 11 + [_P]),
    "conv2d_bwd_data": (_I, [_I, _P, _P, _P] + [_I] * 11 + [_P]),
    "conv2d_bwd_filter_workspace_size": (_Z, [_I] * 12),
    "conv2d_bwd_filter": (_I, [_I, _P, _P, _P, _P, _Z] + [_I] * 11 + [_P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_version": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m attention_forward_backward_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_symbols() -> list[str]:
    """Function names declared in include/attn.h and include/conv.h."""
    names = set()
    for path in (HEADER_PATH, CONV_HEADER_PATH):
        with open(path) as f:
            text = f.read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?((?:attn|conv2d)_\w+)\s*\(",
                                text, re.M))
    return sorted(names)


def attn_status_string(code: int) -> str:
    return lib().attn_status_string(code).decode()


def attn_version() -> str:
    return lib().attn_version().decode()


# ---------------------------------------------------------------- torch marshalling
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"attention tensors must be float32 or bfloat16, got {t.dtype}")


def _check(tensors: dict, shape, dtype) -> None:
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_f32(tensors: dict, shape) -> None:
    import torch
    _check(tensors, shape, torch.float32)


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _raise(func: str, code: int) -> None:
    if code != 0:
        raise AttnError(func, code)


def attn_bwd_workspace_size(dtype: int, batch: int, heads: int, seq: int, head_dim: int,
                            causal: bool) -> int:
    return int(lib().attn_bwd_workspace_size(dtype, batch, heads, seq, head_dim, int(causal)))


def attn_bwd_workspace_size_min(dtype: int, batch: int, heads: int, seq: int, head_dim: int,
                                causal: bool) -> int:
    return int(lib().attn_bwd_workspace_size_min(dtype, batch, heads, seq, head_dim, int(causal)))


def attn_bwd_cross_workspace_size(dtype: int, batch: int, heads: int, seq_q: int, seq_k: int,
                                  head_dim: int, causal: bool) -> int:
    return int(lib().attn_bwd_cross_workspace_size(dtype, batch, heads, seq_q, seq_k, head_dim,
                                                   int(causal)))


def attn_bwd_cross_workspace_size_min(dtype: int, batch: int, heads: int, seq_q: int, seq_k: int,
                                      head_dim: int, causal: bool) -> int:
    return int(lib().attn_bwd_cross_workspace_size_min(dtype, batch, heads, seq_q, seq_k,
                                                       head_dim, int(causal)))


def _kv_len_ptr(kv_len, batch: int) -> int:
    import torch
    if kv_len is None:
        return 0
    if not kv_len.is_cuda or kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (batch,) \
            or not kv_len.is_contiguous():
        raise ValueError(f"kv_len must be a contiguous int32 device tensor of shape ({batch},)")
    return kv_len.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def attn_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None,
             bf16_operands: bool = False) -> None:
    """O, LSE <- attention(Q, K, V); tensors [B,H,S,D] (LSE [B,H,S] float32).

    lse=None: inference-only forward (no LSE stored).  bf16_operands=True with
    float32 tensors selects ATTN_F32_BF16FWD (operands rounded to bf16 inside
    the kernel, f32 accumulation and stores)."""
    B, H, S, D = q.shape
    _check({"q": q, "k": k, "v": v, "o": o}, (B, H, S, D), q.dtype)
    if lse is not None:
        _check_f32({"lse": lse}, (B, H, S))
    code = _dtype_code(q)
    if bf16_operands:
        if code != ATTN_F32:
            raise TypeError("bf16_operands applies to float32 tensors")
        code = ATTN_F32_BF16FWD
    code = lib().attn_fwd(code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          o.data_ptr(), 0 if lse is None else lse.data_ptr(), B, H, S, D,
                          int(causal), float(scale), _stream(stream))
    _raise("attn_fwd", code)


def attn_fwd_workspace_size(code: int, B: int, H: int, S: int, D: int, causal: bool) -> int:
    """Bytes of workspace for the key-split forward (0: the shape is not split)."""
    return int(lib().attn_fwd_workspace_size(code, B, H, S, D, int(causal)))


def attn_fwd_ws(q, k, v, o, lse, workspace, causal: bool, scale: float, stream=None,
                bf16_operands: bool = False) -> None:
    """attn_fwd with a workspace (a device tensor, or None): the key split is
    used when the workspace holds attn_fwd_workspace_size() bytes."""
    B, H, S, D = q.shape
    _check({"q": q, "k": k, "v": v, "o": o}, (B, H, S, D), q.dtype)
    if lse is not None:
        _check_f32({"lse": lse}, (B, H, S))
    code = _dtype_code(q)
    if bf16_operands:
        if code != ATTN_F32:
            raise TypeError("bf16_operands applies to float32 tensors")
        code = ATTN_F32_BF16FWD
    code = lib().attn_fwd_ws(code, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             0 if lse is None else lse.data_ptr(),
                             0 if workspace is None else workspace.data_ptr(),
                             0 if workspace is None else _nbytes(workspace), B, H, S, D,
                             int(causal), float(scale), _stream(stream))
    _raise("attn_fwd_ws", code)


def attn_fwd_cross(q, k, v, o, lse, kv_len, causal: bool, scale: float, stream=None,
                   bf16_operands: bool = False) -> None:
    """Cross-attention forward: q, o [B,H,Sq,D]; k, v [B,H,Sk,D]; lse [B,H,Sq] or
    None; kv_len None or an int32 device tensor [B] of valid keys per batch."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    _check({"q": q, "o": o}, (B, H, Sq, D), q.dtype)
    _check({"k": k, "v": v}, (B, H, Sk, D), q.dtype)
    if lse is not None:
        _check_f32({"lse": lse}, (B, H, Sq))
    code = _dtype_code(q)
    if bf16_operands:
        if code != ATTN_F32:
            raise TypeError("bf16_operands applies to float32 tensors")
        code = ATTN_F32_BF16FWD
    code = lib().attn_fwd_cross(code, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                0 if lse is None else lse.data_ptr(), B, H, Sq, Sk, D,
                                _kv_len_ptr(kv_len, B), int(causal), float(scale),
                                _stream(stream))
    _raise("attn_fwd_cross", code)


def attn_bwd_cross(q, k, v, o, dout, lse, dq, dk, dv, workspace, kv_len, causal: bool,
                   scale: float, stream=None) -> None:
    """Cross-attention backward (shapes as attn_fwd_cross; dq like q, dk and dv like k)."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    _check({"q": q, "o": o, "dout": dout, "dq": dq}, (B, H, Sq, D), q.dtype)
    _check({"k": k, "v": v, "dk": dk, "dv": dv}, (B, H, Sk, D), q.dtype)
    _check_f32({"lse": lse}, (B, H, Sq))
    code = lib().attn_bwd_cross(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                _nbytes(workspace), B, H, Sq, Sk, D, _kv_len_ptr(kv_len, B),
                                int(causal), float(scale), _stream(stream))
    _raise("attn_bwd_cross", code)


def _view_strides(tensors: dict, shape, dtype) -> list:
    """(batch, head, row) element strides of [B,H,S,D] views whose last
    dimension is contiguous (any view torch can make lies inside its
    storage, so the strides address only the tensor's own memory)."""
    out = []
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
        out.extend(int(x) for x in t.stride()[:3])
    return out


def attn_fwd_strided(q, k, v, o, lse, kv_len, causal: bool, scale: float, stream=None,
                     bf16_operands: bool = False) -> None:
    """attn_fwd_cross on [B,H,S,D] views of any layout with a contiguous head
    dimension (e.g. slices of a packed [B,S,3,H,D] projection, permuted
    [B,S,H,D] tensors); lse [B,H,Sq] contiguous float32 or None."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    st = _view_strides({"q": q}, (B, H, Sq, D), q.dtype) + \
        _view_strides({"k": k, "v": v}, (B, H, Sk, D), q.dtype) + \
        _view_strides({"o": o}, (B, H, Sq, D), q.dtype)
    if lse is not None:
        _check_f32({"lse": lse}, (B, H, Sq))
    code = _dtype_code(q)
    if bf16_operands:
        if code != ATTN_F32:
            raise TypeError("bf16_operands applies to float32 tensors")
        code = ATTN_F32_BF16FWD
    code = lib().attn_fwd_strided(code, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  0 if lse is None else lse.data_ptr(), B, H, Sq, Sk, D,
                                  _kv_len_ptr(kv_len, B), (ctypes.c_longlong * 12)(*st),
                                  int(causal), float(scale), _stream(stream))
    _raise("attn_fwd_strided", code)


def attn_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, workspace, kv_len, causal: bool,
                     scale: float, stream=None) -> None:
    """attn_bwd_cross on [B,H,S,D] views (as attn_fwd_strided); the
    workspace is contiguous, sized by attn_bwd_cross_workspace_size."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    qs, ks = (B, H, Sq, D), (B, H, Sk, D)
    st = []
    for name, t, shp in (("q", q, qs), ("k", k, ks), ("v", v, ks), ("o", o, qs),
                         ("dout", dout, qs), ("dq", dq, qs), ("dk", dk, ks), ("dv", dv, ks)):
        st += _view_strides({name: t}, shp, q.dtype)
    _check_f32({"lse": lse}, (B, H, Sq))
    code = lib().attn_bwd_strided(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                  dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                  _nbytes(workspace), B, H, Sq, Sk, D, _kv_len_ptr(kv_len, B),
                                  (ctypes.c_longlong * 24)(*st), int(causal), float(scale),
                                  _stream(stream))
    _raise("attn_bwd_strided", code)


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
             stream=None) -> None:
    """dQ, dK, dV <- attention backward; workspace is a device tensor of at
    least attn_bwd_workspace_size() bytes."""
    B, H, S, D = q.shape
    _check({"q": q, "k": k, "v": v, "o": o, "dout": dout, "dq": dq, "dk": dk, "dv": dv},
           (B, H, S, D), q.dtype)
    _check_f32({"lse": lse}, (B, H, S))
    code = lib().attn_bwd(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                          dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                          _nbytes(workspace), B, H, S, D,
                          int(causal), float(scale), _stream(stream))
    _raise("attn_bwd", code)


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float,
                     stream=None) -> None:
    """dQ, dK, dV <- attention backward with the library's own device scratch
    as the workspace (no workspace argument; calls on one GPU must not
    overlap)."""
    B, H, S, D = q.shape
    _check({"q": q, "k": k, "v": v, "o": o, "dout": dout, "dq": dq, "dk": dk, "dv": dv},
           (B, H, S, D), q.dtype)
    _check_f32({"lse": lse}, (B, H, S))
    code = lib().attn_bwd_noalloc(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                  dk.data_ptr(), dv.data_ptr(), B, H, S, D,
                                  int(causal), float(scale), _stream(stream))
    _raise("attn_bwd_noalloc", code)


def attn_bwd_prep(o, dout, lse, workspace, stream=None) -> None:
    B, H, S, D = o.shape
    _check({"o": o, "dout": dout}, (B, H, S, D), o.dtype)
    _check_f32({"lse": lse}, (B, H, S))
    code = lib().attn_bwd_prep(_dtype_code(o), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                               workspace.data_ptr(), _nbytes(workspace), B, H, S, D,
                               _stream(stream))
    _raise("attn_bwd_prep", code)


def attn_bwd_dkdv(q, k, v, dout, dk, dv, workspace, causal: bool, scale: float,
                  stream=None) -> None:
    B, H, S, D = q.shape
    _check({"q": q, "k": k, "v": v, "dout": dout, "dk": dk, "dv": dv}, (B, H, S, D), q.dtype)
    code = lib().attn_bwd_dkdv(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               dout.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                               _nbytes(workspace), B, H, S, D, int(causal), float(scale),
                               _stream(stream))
    _raise("attn_bwd_dkdv", code)


def attn_bwd_dq(q, k, v, dout, dq, workspace, causal: bool, scale: float, stream=None) -> None:
    B, H, S, D = q.shape
    _check({"q": q, "k": k, "v": v, "dout": dout, "dq": dq}, (B, H, S, D), q.dtype)
    code = lib().attn_bwd_dq(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             dout.data_ptr(), dq.data_ptr(), workspace.data_ptr(),
                             _nbytes(workspace), B, H, S, D, int(causal), float(scale),
                             _stream(stream))
    _raise("attn_bwd_dq", code)


# ---------------------------------------------------------------- layouts, RoPE
def strides_bhsd(heads: int, seq: int, head_dim: int) -> tuple:
    """Element strides (batch, head, row) of a [B, H, S, D] row-major tensor."""
    return (heads * seq * head_dim, seq * head_dim, head_dim)


def strides_bshd(heads: int, seq: int, head_dim: int) -> tuple:
    """Element strides (batch, head, row) of a [B, S, H, D] row-major tensor."""
    return (seq * heads * head_dim, head_dim, heads * head_dim)


def packed_qkv(heads: int, seq: int, head_dim: int) -> tuple:
    """(offsets of Q, K, V, strides) inside a packed [B, S, 3, H, D] tensor."""
    hd = heads * head_dim
    return (0, hd, 2 * hd), (seq * 3 * hd, head_dim, 3 * hd)


def _max_row_start(shape, offset: int, strides) -> int:
    B, H, S, _ = shape
    return offset + sum(st * (n - 1) for st, n in zip(strides, (B, H, S)))


def attn_rope_copy(src, src_offset: int, src_strides, dst, dst_offset: int, dst_strides, shape,
                   cos=None, sin=None, pos_offset: int = 0, transpose: bool = False,
                   stream=None) -> None:
    """Rows (b, h, s) of src -> rows of dst, each head_dim contiguous elements
    at offset + b*strides[0] + h*strides[1] + s*strides[2] of the flat tensor;
    rotated by the [P, head_dim/2] float32 cos/sin tables (table row
    pos_offset + s), by their transpose with transpose=True, or copied when
    no tables are given.  Every addressed row is checked to lie inside its
    tensor before the call."""
    import torch
    B, H, S, D = (int(x) for x in shape)
    for name, t, off, st in (("src", src, src_offset, src_strides),
                             ("dst", dst, dst_offset, dst_strides)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if off < 0 or min(st) < 0:
            raise ValueError(f"{name}: negative offset or stride")
        if _max_row_start((B, H, S, D), off, st) + D > t.numel():
            raise ValueError(f"{name}: rows reach past the end of the tensor")
    if src.dtype != dst.dtype:
        raise ValueError("src and dst must have the same dtype")
    code = _dtype_code(src)
    rows = 0
    cp = sp = 0
    if (cos is None) != (sin is None):
        raise ValueError("give both tables or neither")
    if cos is not None:
        for name, t in (("cos", cos), ("sin", sin)):
            if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() \
                    or t.dim() != 2 or t.shape[1] != D // 2:
                raise ValueError(f"{name} must be a contiguous float32 device tensor [P, {D // 2}]")
        if cos.shape != sin.shape:
            raise ValueError("cos and sin tables differ in shape")
        rows, cp, sp = int(cos.shape[0]), cos.data_ptr(), sin.data_ptr()
    LL3 = ctypes.c_longlong * 3
    esz = src.element_size()
    code = lib().attn_rope_copy(code, src.data_ptr() + src_offset * esz, LL3(*src_strides),
                                dst.data_ptr() + dst_offset * esz, LL3(*dst_strides), cp, sp,
                                rows, int(pos_offset), B, H, S, D, int(bool(transpose)),
                                _stream(stream))
    _raise("attn_rope_copy", code)


def _rope_tables(cos, sin, half: int):
    import torch
    for name, t in (("cos", cos), ("sin", sin)):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() \
                or t.dim() != 2 or t.shape[1] != half:
            raise ValueError(f"{name} must be a contiguous float32 device tensor [P, {half}]")
    if cos.shape != sin.shape:
        raise ValueError("cos and sin tables differ in shape")
    return int(cos.shape[0]), cos.data_ptr(), sin.data_ptr()


def _check_qk_rot(qk_rot, shape, dtype):
    B, H, S, D = shape
    if not qk_rot.is_cuda or not qk_rot.is_contiguous() or qk_rot.dtype != dtype \
            or qk_rot.numel() != 2 * B * H * S * D:
        raise ValueError(f"qk_rot must be a contiguous {dtype} device tensor of "
                         f"2*B*H*S*D = {2 * B * H * S * D} elements")


def attn_fwd_rope(q, k, v, o, lse, qk_rot, cos, sin, causal: bool, scale: float,
                  pos_offset: int = 0, stream=None, bf16_operands: bool = False) -> None:
    """Self-attention forward with RoPE on Q and K fused into the kernels:
    q, k, v, o are [B,H,S,D] views of any layout with a contiguous head
    dimension (as attn_fwd_strided); cos, sin [P, D/2] float32 tables (query
    and key i at row pos_offset + i); qk_rot a [2, B, H, S, D] tensor of the
    inputs' dtype that receives the turned Q and K for attn_bwd_rope."""
    B, H, S, D = q.shape
    st = _view_strides({"q": q, "k": k, "v": v, "o": o}, (B, H, S, D), q.dtype)
    _check_qk_rot(qk_rot, (B, H, S, D), q.dtype)
    if lse is not None:
        _check_f32({"lse": lse}, (B, H, S))
    rows, cp, sp = _rope_tables(cos, sin, D // 2)
    code = _dtype_code(q)
    if bf16_operands:
        if code != ATTN_F32:
            raise TypeError("bf16_operands applies to float32 tensors")
        code = ATTN_F32_BF16FWD
    code = lib().attn_fwd_rope(code, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               0 if lse is None else lse.data_ptr(), qk_rot.data_ptr(), B, H, S, D,
                               (ctypes.c_longlong * 12)(*st), cp, sp, rows, int(pos_offset),
                               int(causal), float(scale), _stream(stream))
    _raise("attn_fwd_rope", code)


def attn_bwd_rope(qk_rot, v, o, dout, lse, dq, dk, dv, workspace, cos, sin, causal: bool,
                  scale: float, pos_offset: int = 0, stream=None) -> None:
    """Backward of attn_fwd_rope: reads the turned Q and K from qk_rot,
    writes dQ and dK with respect to the unturned inputs (and dV) into
    [B,H,S,D] views of any layout with a contiguous head dimension; the
    workspace is sized by attn_bwd_workspace_size."""
    B, H, S, D = v.shape
    st = _view_strides({"v": v, "o": o, "dout": dout, "dq": dq, "dk": dk, "dv": dv},
                       (B, H, S, D), v.dtype)
    _check_qk_rot(qk_rot, (B, H, S, D), v.dtype)
    _check_f32({"lse": lse}, (B, H, S))
    rows, cp, sp = _rope_tables(cos, sin, D // 2)
    code = lib().attn_bwd_rope(_dtype_code(v), qk_rot.data_ptr(), v.data_ptr(), o.data_ptr(),
                               dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), workspace.data_ptr(), _nbytes(workspace), B, H, S,
                               D, (ctypes.c_longlong * 18)(*st), cp, sp, rows, int(pos_offset),
                               int(causal), float(scale), _stream(stream))
    _raise("attn_bwd_rope", code)


# ---------------------------------------------------------------- convolution (include/conv.h)
def conv2d_out_size(height: int, width: int, kh: int, kw: int, stride, pad) -> tuple:
    """(P, Q) of the convolution output (rounded down)."""
    return ((height + 2 * pad[0] - kh) // stride[0] + 1, (width + 2 * pad[1] - kw) // stride[1] + 1)


def _conv_dims(x_shape, w_shape, stride, pad) -> list:
    N, H, W, C = x_shape
    K, R, S, C2 = w_shape
    if C != C2:
        raise ValueError(f"x has {C} channels, w {C2}")
    return [N, H, W, C, K, R, S, int(stride[0]), int(stride[1]), int(pad[0]), int(pad[1])]


def conv2d_fwd(x, w, y, stride=(1, 1), pad=(0, 0), stream=None) -> None:
    """y [N,P,Q,K] = conv(x [N,H,W,C], w [K,R,S,C]) (include/conv.h)."""
    dims = _conv_dims(x.shape, w.shape, stride, pad)
    P, Q = conv2d_out_size(dims[1], dims[2], dims[5], dims[6], stride, pad)
    _check({"x": x}, x.shape, x.dtype)
    _check({"w": w}, w.shape, x.dtype)
    _check({"y": y}, (dims[0], P, Q, dims[4]), x.dtype)
    _raise("conv2d_fwd", lib().conv2d_fwd(_dtype_code(x), x.data_ptr(), w.data_ptr(),
                                          y.data_ptr(), *dims, _stream(stream)))


def conv2d_bwd_data(dy, w, dx, stride=(1, 1), pad=(0, 0), stream=None) -> None:
    """dx [N,H,W,C] from dy [N,P,Q,K] and w [K,R,S,C] (include/conv.h)."""
    dims = _conv_dims(dx.shape, w.shape, stride, pad)
    P, Q = conv2d_out_size(dims[1], dims[2], dims[5], dims[6], stride, pad)
    _check({"dx": dx}, dx.shape, dx.dtype)
    _check({"w": w}, w.shape, dx.dtype)
    _check({"dy": dy}, (dims[0], P, Q, dims[4]), dx.dtype)
    _raise("conv2d_bwd_data", lib().conv2d_bwd_data(_dtype_code(dx), dy.data_ptr(), w.data_ptr(),
                                                    dx.data_ptr(), *dims, _stream(stream)))


def conv2d_bwd_filter_workspace_size(dtype: int, x_shape, w_shape, stride=(1, 1),
                                     pad=(0, 0)) -> int:
    return int(lib().conv2d_bwd_filter_workspace_size(dtype, *_conv_dims(x_shape, w_shape,
                                                                           stride, pad)))


def conv2d_bwd_filter(x, dy, dw, workspace, stride=(1, 1), pad=(0, 0), stream=None) -> None:
    """dw [K,R,S,C] from x [N,H,W,C] and dy [N,P,Q,K]; workspace: a device
    tensor of at least conv2d_bwd_filter_workspace_size bytes, or None when
    that size is 0 (include/conv.h)."""
    dims = _conv_dims(x.shape, dw.shape, stride, pad)
    P, Q = conv2d_out_size(dims[1], dims[2], dims[5], dims[6], stride, pad)
    _check({"x": x}, x.shape, x.dtype)
    _check({"dw": dw}, dw.shape, x.dtype)
    _check({"dy": dy}, (dims[0], P, Q, dims[4]), x.dtype)
    if workspace is None:
        wp, wb = 0, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        wp, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _raise("conv2d_bwd_filter", lib().conv2d_bwd_filter(_dtype_code(x), x.data_ptr(),
                                                        dy.data_ptr(), dw.data_ptr(), wp, wb,
                                                        *dims, _stream(stream)))
