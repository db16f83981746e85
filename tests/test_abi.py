"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/attn.h declares, and rejects bad arguments before anything
is launched (every call here fails validation, so no kernel ever runs)."""
import ctypes
import math

import pytest

import attention_forward_backward_amd as afb

FAKE = 0x10000          # aligned, non-null; never dereferenced (validation fails first)
MIS = 0x10008           # 8-byte aligned only


def test_library_loads_and_exports_header_symbols():
    L = afb.lib()
    declared = afb.declared_symbols()
    assert set(declared) == {"attn_fwd", "attn_fwd_ws", "attn_fwd_workspace_size", "attn_bwd",
                             "attn_bwd_noalloc", "attn_bwd_prep",
                             "attn_bwd_dq",
                             "attn_bwd_dkdv", "attn_bwd_workspace_size",
                             "attn_bwd_workspace_size_min", "attn_fwd_cross", "attn_bwd_cross",
                             "attn_bwd_cross_workspace_size", "attn_bwd_cross_workspace_size_min",
                             "attn_rope_copy", "attn_fwd_strided", "attn_bwd_strided",
                             "attn_fwd_rope", "attn_bwd_rope",
                             "attn_status_string", "attn_version", "conv2d_fwd",
                             "conv2d_bwd_data", "conv2d_bwd_filter",
                             "conv2d_bwd_filter_workspace_size"}
    for name in declared:
        assert hasattr(L, name), name
    assert afb.attn_version() == "0.8.0"
    for code in range(5):
        assert afb.attn_status_string(code) not in ("", "unknown status")
    assert afb.attn_status_string(99) == "unknown status"


def _fwd(dtype=0, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, S=8, D=64, causal=1,
         scale=0.125):
    return afb.lib().attn_fwd(dtype, q, k, v, o, lse, B, H, S, D, causal, scale, None)


def _bwd(dtype=0, ptr=FAKE, ws=FAKE, wsb=1 << 20, B=1, H=1, S=8, D=64, causal=1, scale=0.125,
         misalign=None):
    p = [ptr] * 9
    if misalign is not None:
        p[misalign] = MIS
    return afb.lib().attn_bwd(dtype, *p, ws, wsb, B, H, S, D, causal, scale, None)


def _bwd_noalloc(dtype=0, ptr=FAKE, B=1, H=1, S=8, D=64, causal=1, scale=0.125, misalign=None):
    p = [ptr] * 9
    if misalign is not None:
        p[misalign] = MIS
    return afb.lib().attn_bwd_noalloc(dtype, *p, B, H, S, D, causal, scale, None)


def test_bwd_noalloc_validation():
    """The allocation-free backward validates like attn_bwd and rejects a
    shape whose minimum workspace exceeds its 128 MiB scratch array
    (B*H*S > 2^24 query rows) before touching the GPU."""
    for i in range(9):
        assert _bwd_noalloc(misalign=i) == 1, i
    assert _bwd_noalloc(ptr=None) == 1
    assert _bwd_noalloc(D=96) == 2 and _bwd_noalloc(dtype=5) == 2
    assert _bwd_noalloc(causal=3) == 1 and _bwd_noalloc(scale=math.nan) == 1
    assert _bwd_noalloc(B=1, H=256, S=(1 << 16) + 1) == 3
    assert _bwd_noalloc(B=4, H=64, S=(1 << 16) + 8, D=32) == 3


def test_fwd_key_split_workspace():
    """The key-split forward's workspace: used for few long heads, 0 for
    shapes with enough work items (or rejected ones); a misaligned workspace
    is rejected, a NULL one means the plain forward."""
    L = afb.lib()
    for dt in (0, 1, 2):
        n = L.attn_fwd_workspace_size(dt, 1, 16, 1024, 128, 1)
        # three chunks (of at most 6 of the 16 key tiles: 3/4 of the 9-tile
        # share), (D + 2) floats per row
        assert n == 3 * 16 * 1024 * (128 + 2) * 4, (dt, n)
        assert L.attn_fwd_workspace_size(dt, 8, 12, 512, 64, 1) == 0  # decoder step: not split
        assert L.attn_fwd_workspace_size(dt, 1, 8, 1024, 64, 0) > 0    # non-causal long heads
        assert L.attn_fwd_workspace_size(dt, 1, 2, 2048, 64, 0) == 0   # B*H not a multiple of 8
    assert L.attn_fwd_workspace_size(0, 1, 16, 1024, 48, 1) == 0
    assert L.attn_fwd_workspace_size(0, 1, 16, 1, 128, 1) == 0        # one-query heads
    ws_mis = MIS
    assert L.attn_fwd_ws(0, FAKE, FAKE, FAKE, FAKE, FAKE, ws_mis, 1 << 30, 1, 16, 1024, 128, 1,
                         0.1, None) == 1
    assert L.attn_fwd_ws(0, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 1, 16, 1024, 128, 1,
                         0.1, None) == 1
    assert L.attn_fwd_ws(0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 1, 16, 1024, 128, 1,
                         -0.1, None) == 1


def test_fwd_validation():
    assert _fwd(q=None) == 1
    assert _fwd(lse=MIS) == 1                      # lse may be NULL (no LSE), not misaligned
    assert _fwd(v=MIS) == 1
    assert _fwd(B=0) == 1 and _fwd(H=-1) == 1 and _fwd(S=0) == 1
    assert _fwd(causal=2) == 1
    assert _fwd(scale=math.inf) == 1 and _fwd(scale=math.nan) == 1
    assert _fwd(scale=0.0) == 1 and _fwd(scale=-0.125) == 1
    assert _fwd(D=48) == 2 and _fwd(D=256) == 2 and _fwd(D=16) == 2
    assert _fwd(dtype=7) == 2 and _fwd(dtype=3) == 2
    assert _fwd(dtype=2, D=48) == 2 and _fwd(dtype=2, q=None) == 1   # ATTN_F32_BF16FWD is validated alike
    assert _fwd(B=1 << 16, H=1 << 16) == 1          # B*H beyond int
    assert _fwd(S=1 << 26, D=64) == 1               # S*D beyond int


def test_bwd_validation():
    for i in range(9):
        assert _bwd(misalign=i) == 1, i
    assert _bwd(ptr=None) == 1
    assert _bwd(ws=None) == 1
    assert _bwd(D=96) == 2
    assert _bwd(dtype=3) == 2
    assert _bwd(wsb=2 * 8 * 4 - 1) == 3
    L = afb.lib()
    # split stages validate the same way
    assert L.attn_bwd_prep(0, FAKE, FAKE, FAKE, FAKE, 16, 1, 1, 8, 64, None) == 3
    assert L.attn_bwd_prep(0, FAKE, None, FAKE, FAKE, 1 << 20, 1, 1, 8, 64, None) == 1
    assert L.attn_bwd_prep(0, FAKE, FAKE, FAKE, FAKE, 1 << 20, 1, 1, 8, 48, None) == 2
    assert L.attn_bwd_dq(0, *[FAKE] * 5, FAKE, 16, 1, 1, 8, 64, 1, 0.1, None) == 3
    assert L.attn_bwd_dkdv(0, *[FAKE] * 6, FAKE, 16, 1, 1, 8, 64, 1, 0.1, None) == 3
    assert L.attn_bwd_dq(0, *[FAKE] * 5, None, 1 << 20, 1, 1, 8, 64, 1, 0.1, None) == 1
    assert L.attn_bwd_dkdv(0, *[FAKE] * 6, None, 1 << 20, 1, 1, 8, 64, 1, 0.1, None) == 1
    assert L.attn_bwd_dkdv(0, *[FAKE] * 6, FAKE, 1 << 20, 1, 1, 8, 64, 1, -1.0, None) == 1


def r256(b):
    return (b + 255) // 256 * 256


def test_workspace_size():
    wmin, wfull = afb.attn_bwd_workspace_size_min, afb.attn_bwd_workspace_size
    # minimum: D and LSE*log2(e), two floats per query row, rounded up to 256 bytes
    assert wmin(0, 8, 12, 512, 64, True) == 2 * 8 * 12 * 512 * 4
    assert wmin(1, 1, 1, 1, 64, False) == 256
    assert wmin(0, 32, 8, 197, 64, False) == r256(2 * 32 * 8 * 197 * 4)
    # full: plus dS^T [B*H][Sp][Sp] (Sp = S rounded up to 128) in the element type
    assert wfull(0, 8, 12, 512, 64, True) == 2 * 8 * 12 * 512 * 4 + 8 * 12 * 512 * 512 * 4
    assert wfull(1, 8, 12, 512, 64, True) == 2 * 8 * 12 * 512 * 4 + 8 * 12 * 512 * 512 * 2
    assert wfull(0, 32, 8, 197, 64, False) == r256(2 * 32 * 8 * 197 * 4) + r256(32 * 8 * 256 * 256 * 4)
    # few long heads (B1 H16 S1024 D128 causal: 16 x 16 = 256 (key tile, head)
    # pairs): with f32 tensors the dK, dV partials of a 2-chunk query split
    # follow dS^T; bf16 keeps the unsplit backward
    assert wfull(0, 1, 16, 1024, 128, True) == (2 * 16 * 1024 * 4 + 16 * 1024 * 1024 * 4
                                                + 2 * 2 * 16 * 1024 * 128 * 4)
    assert wfull(1, 1, 16, 1024, 128, True) == 2 * 16 * 1024 * 4 + 16 * 1024 * 1024 * 2
    # the practical contract (bf16 forward operands, strict f32 backward) sizes as f32
    assert wfull(2, 8, 12, 512, 64, True) == wfull(0, 8, 12, 512, 64, True)
    assert wmin(2, 32, 8, 197, 64, False) == wmin(0, 32, 8, 197, 64, False)
    for f in (wmin, wfull):
        assert f(0, 1, 1, 8, 48, True) == 0 and f(0, 0, 1, 8, 64, True) == 0
        assert f(5, 1, 1, 8, 64, True) == 0
    prev = 0
    for s in (1, 17, 64, 197, 512, 1024):
        lo, hi = wmin(0, 2, 3, s, 64, True), wfull(0, 2, 3, s, 64, True)
        assert lo >= 2 * 2 * 3 * s * 4 and lo % 256 == 0 and hi % 256 == 0
        assert hi >= lo + 2 * 3 * s * s * 4 and hi >= prev
        prev = hi


def test_no_cpu_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(afb, "_lib", None)
    monkeypatch.setattr(afb, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        afb.lib()


def _fwdx(dtype=0, q=FAKE, lse=FAKE, B=1, H=1, Sq=8, Sk=16, D=64, kvl=None, causal=1, scale=0.125):
    return afb.lib().attn_fwd_cross(dtype, q, FAKE, FAKE, FAKE, lse, B, H, Sq, Sk, D, kvl, causal,
                                    scale, None)


def test_cross_validation_and_workspace():
    assert _fwdx(Sq=0) == 1 and _fwdx(Sk=0) == 1 and _fwdx(Sk=-3) == 1
    assert _fwdx(q=None) == 1 and _fwdx(lse=MIS) == 1
    assert _fwdx(kvl=FAKE + 2) == 1                      # kv_len must be 4-byte aligned
    assert _fwdx(D=48) == 2 and _fwdx(dtype=3) == 2
    L = afb.lib()
    p = [FAKE] * 10
    assert L.attn_bwd_cross(0, *p, 16, 1, 1, 8, 16, 64, None, 1, 0.1, None) == 3  # workspace
    assert L.attn_bwd_cross(0, *p, 1 << 20, 1, 1, 8, 16, 64, FAKE + 1, 1, 0.1, None) == 1
    assert L.attn_bwd_cross(0, *p[:9], None, 1 << 20, 1, 1, 8, 16, 64, None, 1, 0.1, None) == 1
    wx, wxm = afb.attn_bwd_cross_workspace_size, afb.attn_bwd_cross_workspace_size_min
    # D and LSE*log2(e) per query row; dS^T [B*H][ceil(Sk/128)*128][ceil(Sq/128)*128]
    assert wxm(0, 2, 3, 77, 1024, 64, False) == r256(2 * 2 * 3 * 77 * 4)
    assert wx(0, 2, 3, 77, 1024, 64, False) == r256(2 * 2 * 3 * 77 * 4) + r256(6 * 1024 * 128 * 4)
    assert wx(1, 2, 3, 1, 512, 64, True) == r256(2 * 6 * 1 * 4) + r256(6 * 512 * 128 * 2)
    # many queries over few keys: plus the dK, dV partials of the query split,
    # [2][C][B*H][Sk][D] f32; B2 H8 Sq4096 Sk77: 32 (key tile, head) pairs,
    # 64 query tiles of 64 -> C = 16 chunks of 4 tiles
    assert wx(0, 2, 8, 4096, 77, 64, False) == (r256(2 * 16 * 4096 * 4) + r256(16 * 128 * 4096 * 4)
                                                + r256(2 * 16 * 16 * 77 * 64 * 4))
    assert wx(1, 2, 8, 4096, 77, 64, False) == (r256(2 * 16 * 4096 * 4) + r256(16 * 128 * 4096 * 2)
                                                + r256(2 * 16 * 16 * 77 * 64 * 4))
    assert wxm(0, 2, 8, 4096, 77, 64, False) == r256(2 * 16 * 4096 * 4)
    # equal lengths: the self-attention sizes
    assert wx(0, 8, 12, 512, 512, 64, True) == afb.attn_bwd_workspace_size(0, 8, 12, 512, 64, True)
    assert wx(0, 1, 1, 8, 0, 64, True) == 0 and wxm(0, 1, 1, 0, 8, 64, True) == 0


def _rope(dtype=0, src=FAKE, ss=(64 * 8, 64 * 8, 64), dst=FAKE, ds=(64 * 8, 64 * 8, 64),
          cos=FAKE, sin=FAKE, rows=8, pos=0, B=1, H=1, S=8, D=64, tr=0):
    LL3 = ctypes.c_longlong * 3
    return afb.lib().attn_rope_copy(dtype, src, None if ss is None else LL3(*ss), dst,
                                    None if ds is None else LL3(*ds), cos, sin, rows, pos, B, H,
                                    S, D, tr, None)


def test_rope_copy_validation():
    assert _rope(src=None) == 1 and _rope(dst=MIS) == 1
    assert _rope(ss=None) == 1 and _rope(ds=None) == 1
    assert _rope(ss=(512, 512, 60)) == 1                 # stride not a multiple of 8
    assert _rope(ds=(-512, 512, 64)) == 1                # negative stride
    assert _rope(ss=(1 << 50, 8, 8)) == 1                # beyond the index range
    assert _rope(cos=None) == 1 and _rope(sin=None) == 1  # one table only
    assert _rope(cos=MIS) == 1
    assert _rope(rows=7) == 1 and _rope(pos=1) == 1      # table too short for the rows used
    assert _rope(pos=-1, rows=100) == 1
    assert _rope(tr=2) == 1
    assert _rope(B=0) == 1 and _rope(S=0) == 1
    assert _rope(D=48) == 2 and _rope(dtype=5) == 2


def _fwds(strides, B=2, H=3, Sq=8, Sk=8, D=64, dtype=0, q=FAKE):
    LL = ctypes.c_longlong * 12
    return afb.lib().attn_fwd_strided(dtype, q, FAKE, FAKE, FAKE, FAKE, B, H, Sq, Sk, D, None,
                                      None if strides is None else LL(*strides), 1, 0.125, None)


def _bwds(strides, B=2, H=3, S=8, D=64, wsb=1 << 20):
    LL = ctypes.c_longlong * 24
    return afb.lib().attn_bwd_strided(0, *([FAKE] * 9), FAKE, wsb, B, H, S, S, D, None,
                                      None if strides is None else LL(*strides), 1, 0.125, None)


def test_strided_validation():
    B, H, S, D = 2, 3, 8, 64
    bhsd = [H * S * D, S * D, D]
    bshd = [S * H * D, D, H * D]
    assert _fwds(None) == 1
    assert _fwds(bhsd * 3 + [H * S * D, S * D, D + 4]) == 1        # row stride not a multiple of 8
    assert _fwds(bhsd * 3 + [-8, S * D, D]) == 1                   # negative
    assert _fwds(bhsd * 3 + [H * S * D, S * D, 1 << 25]) == 1      # row stride beyond 2^24
    assert _fwds(bhsd * 3 + [H * S * D, 0, D]) == 1                # output heads overlap
    assert _fwds(bhsd * 3 + [H * S * D, S * D, 32]) == 1           # output rows overlap (32 < D)
    assert _fwds(bhsd * 3 + bhsd, q=None) == 1
    assert _fwds(bhsd * 3 + bhsd, D=48) == 2
    # shared K, V head (head stride 0) is a valid input; overlapping dK is not
    mq = bhsd + [S * D, 0, D] * 2
    assert _bwds(mq + bhsd * 2 + bshd + [S * D, 0, D] * 2) == 1
    assert _bwds(mq + bhsd * 5, wsb=16) == 3                       # workspace still checked


def _fwd_rope(strides=None, qk=FAKE, cos=FAKE, sin=FAKE, rows=8, pos=0, B=2, H=3, S=8, D=64,
              dtype=0, lse=FAKE):
    if strides is None:
        strides = [H * S * D, S * D, D] * 4
    LL = ctypes.c_longlong * 12
    return afb.lib().attn_fwd_rope(dtype, FAKE, FAKE, FAKE, FAKE, lse, qk, B, H, S, D,
                                   LL(*strides), cos, sin, rows, pos, 1, 0.125, None)


def _bwd_rope(strides=None, qk=FAKE, cos=FAKE, sin=FAKE, rows=8, pos=0, B=2, H=3, S=8, D=64,
              wsb=1 << 20):
    if strides is None:
        strides = [H * S * D, S * D, D] * 6
    LL = ctypes.c_longlong * 18
    return afb.lib().attn_bwd_rope(0, qk, *([FAKE] * 7), FAKE, wsb, B, H, S, D, LL(*strides),
                                   cos, sin, rows, pos, 1, 0.125, None)


def test_rope_fused_validation():
    """attn_fwd_rope / attn_bwd_rope reject bad tables, qk_rot and strides
    before the rotation pass or any kernel is enqueued."""
    B, H, S, D = 2, 3, 8, 64
    bhsd = [H * S * D, S * D, D]
    for fn in (_fwd_rope, _bwd_rope):
        assert fn(qk=None) == 1 and fn(qk=MIS) == 1
        assert fn(cos=None) == 1 and fn(sin=None) == 1 and fn(cos=MIS) == 1
        assert fn(rows=7) == 1 and fn(pos=1) == 1 and fn(pos=-1, rows=100) == 1
        assert fn(D=48) == 2
        # heads*seq*head_dim of qk_rot at 2^31 elements (the given strides pass)
        n = 4 if fn is _fwd_rope else 6
        assert fn(B=1, H=256, S=1 << 17, D=64, rows=1 << 17,
                  strides=[0, (1 << 17) * 64, 64] * n) == 1
    assert _fwd_rope(lse=MIS) == 1
    assert _fwd_rope(strides=bhsd * 3 + [H * S * D, S * D, 32]) == 1   # output rows overlap
    assert _bwd_rope(strides=bhsd * 3 + [H * S * D, 0, D] + bhsd * 2) == 1  # dq heads overlap
    assert _bwd_rope(wsb=16) == 3


def _conv(fn, dtype=0, a=FAKE, b=FAKE, out=FAKE, dims=(2, 8, 8, 4, 6, 3, 3, 1, 1, 1, 1)):
    return getattr(afb.lib(), fn)(dtype, a, b, out, *dims, None)


def test_conv_validation():
    L = afb.lib()
    for fn in ("conv2d_fwd", "conv2d_bwd_data"):
        assert _conv(fn, dtype=5) == 2                               # unknown dtype
        assert _conv(fn, dtype=2) == 2                               # practical: not a conv contract
        assert _conv(fn, a=None) == 1 and _conv(fn, out=None) == 1   # null pointers
        assert _conv(fn, a=FAKE + 2) == 1                            # f32 needs 4-byte alignment
        bad = [(0, 8, 8, 4, 6, 3, 3, 1, 1, 1, 1),    # empty batch
               (2, 8, 8, 4, 6, 3, 3, 0, 1, 1, 1),    # zero stride
               (2, 8, 8, 4, 6, 3, 3, 1, 1, -1, 1),   # negative padding
               (2, 2, 8, 4, 6, 5, 3, 1, 1, 1, 1),    # filter taller than the padded image
               (1 << 16, 256, 256, 4, 6, 3, 3, 1, 1, 1, 1)]  # x beyond 2^31 elements
        for d in bad:
            assert _conv(fn, dims=d) == 1, (fn, d)
    ws = L.conv2d_bwd_filter_workspace_size
    # small reductions take one slice and need no workspace; long ones split
    assert ws(0, 1, 4, 4, 2, 3, 3, 3, 1, 1, 1, 1) == 0
    big = (32, 56, 56, 64, 64, 3, 3, 1, 1, 1, 1)
    n32, n16 = ws(0, *big), ws(1, *big)
    assert n32 > 0 and n32 % 256 == 0 and n32 % (64 * 576 * 4) == 0 and n16 == n32
    assert ws(5, *big) == 0 and ws(0, 0, 56, 56, 64, 64, 3, 3, 1, 1, 1, 1) == 0
    args = lambda wsp, wsb: L.conv2d_bwd_filter(0, FAKE, FAKE, FAKE, wsp, wsb, *big, None)
    assert args(None, n32) == 3 and args(FAKE, n32 - 256) == 3 and args(FAKE + 8, n32) == 3
