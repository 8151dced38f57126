"""Host-only checks of the C ABI: the library loads, exports every function
that include/wanvae.h declares, and rejects invalid arguments before it
touches the GPU (argument validation runs on the host before any launch)."""
import ctypes as C
import os
import re

import pytest

import causal_convolution_amd as wv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wanvae.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"WANVAE_API\s+[\w\s\*]+?\b(wanvae_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("wanvae_rmsnorm_silu", "wanvae_causal_conv3d", "wanvae_resblock_forward",
              "wanvae_resblock_stream_step", "wanvae_resblock_workspace_size", "wanvae_last_error"):
        assert f in names


def test_library_exports_every_declared_function():
    L = wv.lib()
    for f in declared_functions():
        assert hasattr(L, f), f
    assert set(declared_functions()) == set(wv.EXPORTS)


def _dims(n=1, t=2, h=3, w=4):
    return wv.Dims(n, t, h, w)


def test_norm_validation():
    L = wv.lib()
    p = C.c_void_p(1 << 20)   # never dereferenced: validation fails first
    assert L.wanvae_rmsnorm_silu(p, p, 10, 33, p, None, 1e-12, wv.BF16, None) == wv.ERR_SHAPE
    assert "multiple of 32" in wv.last_error()
    assert L.wanvae_rmsnorm_silu(p, p, 10, 2048, p, None, 1e-12, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_rmsnorm_silu(p, p, 10, 64, p, None, 1e-12, 9, None) == wv.ERR_DTYPE
    assert L.wanvae_rmsnorm_silu(None, p, 10, 64, p, None, 1e-12, wv.BF16, None) == wv.ERR_NULL
    assert L.wanvae_rmsnorm_silu(p, p, 10, 64, None, None, 1e-12, wv.BF16, None) == wv.ERR_NULL
    assert L.wanvae_rmsnorm_silu(p, p, -1, 64, p, None, 1e-12, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_rmsnorm_silu(p, p, 10, 64, p, None, float("nan"), wv.BF16, None) == wv.ERR_SHAPE
    # partial overlap is an alias error (y == x is allowed)
    q = C.c_void_p((1 << 20) + 64)
    assert L.wanvae_rmsnorm_silu(p, q, 10, 64, p, None, 1e-12, wv.BF16, None) == wv.ERR_ALIAS
    # misaligned pointer
    m = C.c_void_p((1 << 20) + 2)
    assert L.wanvae_rmsnorm_silu(m, m, 10, 64, p, None, 1e-12, wv.BF16, None) == wv.ERR_SHAPE
    # empty input: nothing to do, no pointer needed
    assert L.wanvae_rmsnorm_silu(None, None, 0, 64, None, None, 1e-12, wv.BF16, None) == wv.OK
    assert wv.last_error() == ""


def test_conv_validation():
    L = wv.lib()
    p = C.c_void_p(1 << 24)
    d = _dims()
    assert L.wanvae_causal_conv3d(p, None, p, None, p, C.byref(d), 24, 64, wv.BF16, None) == wv.ERR_SHAPE
    assert "multiple of 16" in wv.last_error()
    assert L.wanvae_causal_conv3d(p, None, p, None, p, C.byref(d), 64, 0, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_causal_conv3d(p, None, p, None, p, C.byref(d), 64, 1025, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_causal_conv3d(p, None, p, None, p, C.byref(d), 64, 2048, wv.F32, None) == wv.ERR_SHAPE
    assert L.wanvae_causal_conv3d(p, None, p, None, p, None, 64, 64, wv.BF16, None) == wv.ERR_NULL
    assert L.wanvae_causal_conv3d(None, None, p, None, p, C.byref(d), 64, 64, wv.BF16, None) == wv.ERR_NULL
    neg = _dims(1, -1, 3, 4)
    assert L.wanvae_causal_conv3d(p, None, p, None, p, C.byref(neg), 64, 64, wv.BF16, None) == wv.ERR_SHAPE
    huge = _dims(1 << 40, 1 << 40, 4, 4)
    assert L.wanvae_causal_conv3d(p, None, p, None, p, C.byref(huge), 64, 64, wv.BF16, None) == wv.ERR_SHAPE
    # y == x is not allowed for the conv
    assert L.wanvae_causal_conv3d(p, None, C.c_void_p(1 << 30), None, p, C.byref(d), 64, 64, wv.BF16,
                                  None) == wv.ERR_ALIAS
    empty = _dims(1, 0, 3, 4)
    assert L.wanvae_causal_conv3d(None, None, None, None, None, C.byref(empty), 64, 64, wv.BF16,
                                  None) == wv.OK


def test_packed_weight_elems():
    L = wv.lib()
    n = C.c_int64(0)
    assert L.wanvae_packed_conv3d_weight_elems(96, 3, wv.BF16, C.byref(n)) == wv.OK
    assert n.value == 27 * 96 * 32                 # bf16: C_out padded to the 32-channel block
    assert L.wanvae_packed_conv3d_weight_elems(16, 384, wv.BF16, C.byref(n)) == wv.OK
    assert n.value == 27 * 16 * 384
    assert L.wanvae_packed_conv3d_weight_elems(3, 5, wv.F32, C.byref(n)) == wv.OK
    assert n.value == 27 * 3 * 5                   # fp32: no padding
    assert L.wanvae_packed_conv3d_weight_elems(24, 3, wv.BF16, C.byref(n)) == wv.ERR_SHAPE
    assert L.wanvae_packed_conv3d_weight_elems(16, 0, wv.BF16, C.byref(n)) == wv.ERR_SHAPE
    assert L.wanvae_packed_conv3d_weight_elems(16, 3, 5, C.byref(n)) == wv.ERR_DTYPE
    assert L.wanvae_packed_conv3d_weight_elems(16, 3, wv.BF16, None) == wv.ERR_NULL


def test_pointwise_validation():
    L = wv.lib()
    p, q = C.c_void_p(1 << 24), C.c_void_p(1 << 30)
    assert L.wanvae_pointwise_conv(p, p, None, q, 10, 65, 16, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_pointwise_conv(p, p, None, q, 10, 16, 0, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_pointwise_conv(p, p, None, q, -1, 16, 16, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_pointwise_conv(p, p, None, q, 10, 16, 16, 3, None) == wv.ERR_DTYPE
    assert L.wanvae_pointwise_conv(None, p, None, q, 10, 16, 16, wv.BF16, None) == wv.ERR_NULL
    assert L.wanvae_pointwise_conv(p, p, None, C.c_void_p((1 << 30) + 2), 10, 16, 16, wv.BF16,
                                   None) == wv.ERR_SHAPE
    # y may not overlap x
    assert L.wanvae_pointwise_conv(p, q, None, C.c_void_p((1 << 24) + 16), 10, 16, 16, wv.BF16,
                                   None) == wv.ERR_ALIAS
    assert L.wanvae_pointwise_conv(None, None, None, None, 0, 16, 16, wv.BF16, None) == wv.OK


def test_pack_validation():
    L = wv.lib()
    p, q = C.c_void_p(1 << 24), C.c_void_p(1 << 30)
    assert L.wanvae_pack_conv3d_weights(p, q, 64, 64, 7, None) == wv.ERR_DTYPE
    assert L.wanvae_pack_conv3d_weights(p, q, 24, 64, wv.BF16, None) == wv.ERR_SHAPE   # cin % 16
    assert L.wanvae_pack_conv3d_weights(p, q, 64, 0, wv.BF16, None) == wv.ERR_SHAPE
    assert L.wanvae_pack_conv3d_weights(p, q, 2048, 64, wv.F32, None) == wv.ERR_SHAPE
    assert L.wanvae_pack_conv3d_weights(None, q, 64, 64, wv.BF16, None) == wv.ERR_NULL
    assert L.wanvae_pack_conv3d_weights(p, C.c_void_p((1 << 30) + 4), 64, 64, wv.BF16, None) == wv.ERR_SHAPE
    # the packed buffer may not overlap the source
    assert L.wanvae_pack_conv3d_weights(p, C.c_void_p((1 << 24) + 4096), 64, 64, wv.BF16, None) == wv.ERR_ALIAS
    assert "overlap" in wv.last_error()


def _params(cin=384, cout=192, dtype=wv.BF16, shortcut=True):
    a = 1 << 24
    vals = [a + i * (1 << 20) for i in range(10)]
    p = wv.ResblockParamsC(cin, cout, dtype, 1e-12, *vals)
    if not shortcut:
        p.w_sc = None
        p.b_sc = None
    return p


def test_workspace_size():
    L = wv.lib()
    b = C.c_size_t(0)
    d = wv.Dims(1, 41, 180, 320)
    p = _params()
    assert L.wanvae_resblock_workspace_size(C.byref(p), C.byref(d), C.byref(b)) == wv.OK
    P = 41 * 180 * 320
    assert b.value >= P * (384 + 192) * 2 and b.value < P * (384 + 192) * 2 + 1024
    assert b.value % 256 == 0
    # the conv input region holds n1 and later n2: max(in_dim, out_dim) per position
    pw = _params(cin=96, cout=192)
    assert L.wanvae_resblock_workspace_size(C.byref(pw), C.byref(d), C.byref(b)) == wv.OK
    assert b.value >= P * (192 + 192) * 2 and b.value < P * (192 + 192) * 2 + 1024
    # identity shortcut with in != out is rejected
    p2 = _params(shortcut=False)
    assert L.wanvae_resblock_workspace_size(C.byref(p2), C.byref(d), C.byref(b)) == wv.ERR_SHAPE
    assert "identity" in wv.last_error()
    p3 = _params(cin=100)
    assert L.wanvae_resblock_workspace_size(C.byref(p3), C.byref(d), C.byref(b)) == wv.ERR_SHAPE
    p4 = _params()
    p4.gamma1 = None
    assert L.wanvae_resblock_workspace_size(C.byref(p4), C.byref(d), C.byref(b)) == wv.ERR_NULL
    assert L.wanvae_resblock_workspace_size(None, C.byref(d), C.byref(b)) == wv.ERR_NULL


def test_forward_and_stream_validation():
    L = wv.lib()
    p = _params()
    d = wv.Dims(1, 2, 8, 32)
    x, y, ws = C.c_void_p(1 << 34), C.c_void_p(1 << 35), C.c_void_p(1 << 36)
    need = C.c_size_t(0)
    assert L.wanvae_resblock_workspace_size(C.byref(p), C.byref(d), C.byref(need)) == wv.OK
    assert L.wanvae_resblock_forward(C.byref(p), x, y, C.byref(d), ws, need.value - 1,
                                     None) == wv.ERR_WORKSPACE
    assert L.wanvae_resblock_forward(C.byref(p), x, y, C.byref(d), None, need.value,
                                     None) == wv.ERR_WORKSPACE
    assert L.wanvae_resblock_forward(C.byref(p), x, x, C.byref(d), ws, need.value,
                                     None) == wv.ERR_ALIAS
    assert L.wanvae_resblock_forward(C.byref(p), x, y, C.byref(d), x, need.value,
                                     None) == wv.ERR_ALIAS
    assert L.wanvae_resblock_forward(C.byref(p), None, y, C.byref(d), ws, need.value,
                                     None) == wv.ERR_NULL
    ca, cb = C.c_void_p(1 << 37), C.c_void_p(1 << 38)
    assert L.wanvae_resblock_stream_step(C.byref(p), x, y, C.byref(d), None, cb, ws, need.value,
                                         None) == wv.ERR_NULL
    assert L.wanvae_resblock_stream_step(C.byref(p), x, y, C.byref(d), ca, ca, ws, need.value,
                                         None) == wv.ERR_ALIAS
    assert L.wanvae_resblock_stream_step(C.byref(p), x, y, C.byref(d), ca, x, ws, need.value,
                                         None) == wv.ERR_ALIAS
    empty = wv.Dims(1, 0, 8, 32)
    assert L.wanvae_resblock_forward(C.byref(p), None, None, C.byref(empty), None, 0, None) == wv.OK


def test_timing_kind_validation():
    L = wv.lib()
    n, ms = C.c_int64(0), C.c_double(0)
    assert L.wanvae_timing_read(99, C.byref(n), C.byref(ms)) == wv.ERR_SHAPE
    assert L.wanvae_timing_read(0, None, C.byref(ms)) == wv.ERR_NULL


def test_attention_validation():
    L = wv.lib()
    ptr = 1 << 24
    d = wv.Dims(1, 2, 8, 32)
    b = C.c_size_t(0)
    p = wv.AttentionParamsC(384, 1e-12, ptr, None, ptr + (1 << 20), None, ptr + (2 << 20), None)
    assert L.wanvae_attention_workspace_size(C.byref(p), C.byref(d), C.byref(b)) == wv.OK
    P, HWp = 2 * 8 * 32, 256
    assert b.value >= P * 384 * 2 * 5 + 2 * 384 * HWp * 2 - P * 384 * 2   # u, qkv, v^T, o
    bad = wv.AttentionParamsC(96, 1e-12, ptr, None, ptr, None, ptr, None)
    assert L.wanvae_attention_workspace_size(C.byref(bad), C.byref(d), C.byref(b)) == wv.ERR_SHAPE
    nul = wv.AttentionParamsC(384, 1e-12, None, None, ptr, None, ptr, None)
    assert L.wanvae_attention_workspace_size(C.byref(nul), C.byref(d), C.byref(b)) == wv.ERR_NULL
    x, y, ws = C.c_void_p(1 << 34), C.c_void_p(1 << 35), C.c_void_p(1 << 36)
    need = C.c_size_t(0)
    assert L.wanvae_attention_workspace_size(C.byref(p), C.byref(d), C.byref(need)) == wv.OK
    assert L.wanvae_attention_block(C.byref(p), x, y, C.byref(d), ws, need.value - 1, None) == wv.ERR_WORKSPACE
    assert L.wanvae_attention_block(C.byref(p), x, x, C.byref(d), ws, need.value, None) == wv.ERR_ALIAS
    assert L.wanvae_attention_block(C.byref(p), None, y, C.byref(d), ws, need.value, None) == wv.ERR_NULL
    empty = wv.Dims(1, 0, 8, 32)
    assert L.wanvae_attention_block(C.byref(p), None, None, C.byref(empty), None, 0, None) == wv.OK


def test_upsample2d_validation():
    L = wv.lib()
    p, q = C.c_void_p(1 << 24), C.c_void_p(1 << 34)
    d = _dims()
    up = L.wanvae_upsample2d_conv
    assert up(p, p, None, q, C.byref(d), 64, 32, wv.F32, None) == wv.ERR_DTYPE     # bf16 only
    assert up(p, p, None, q, C.byref(d), 64, 32, 5, None) == wv.ERR_DTYPE
    assert up(p, p, None, q, C.byref(d), 24, 32, wv.BF16, None) == wv.ERR_SHAPE    # cin % 16
    assert up(p, p, None, q, C.byref(d), 64, 0, wv.BF16, None) == wv.ERR_SHAPE
    assert up(p, p, None, q, C.byref(d), 64, 1025, wv.BF16, None) == wv.ERR_SHAPE
    assert up(p, p, None, q, None, 64, 32, wv.BF16, None) == wv.ERR_NULL
    assert up(None, p, None, q, C.byref(d), 64, 32, wv.BF16, None) == wv.ERR_NULL
    assert up(p, p, None, C.c_void_p((1 << 34) + 8), C.byref(d), 64, 32, wv.BF16, None) == wv.ERR_SHAPE
    # the output frame (2h x 2w x cout) must stay below 2 GiB
    big = _dims(1, 1, 4096, 4096)
    assert up(p, p, None, q, C.byref(big), 64, 32, wv.BF16, None) == wv.ERR_SHAPE
    # y may not overlap x (x: 1*2*3*4*64*2 = 3 KB from 1 << 24)
    assert up(p, q, None, C.c_void_p((1 << 24) + 1024), C.byref(d), 64, 32, wv.BF16, None) == wv.ERR_ALIAS
    empty = _dims(0, 2, 3, 4)
    assert up(None, None, None, None, C.byref(empty), 64, 32, wv.BF16, None) == wv.OK
    n = C.c_int64(0)
    # C_out a multiple of 96: 4 output phases x 4 merged taps; otherwise the 9 taps
    assert L.wanvae_packed_conv2d_weight_elems(384, 192, wv.BF16, C.byref(n)) == wv.OK
    assert n.value == 16 * 384 * 192
    assert L.wanvae_packed_conv2d_weight_elems(64, 128, wv.BF16, C.byref(n)) == wv.OK
    assert n.value == 9 * 64 * 128
    assert L.wanvae_packed_conv2d_weight_elems(192, 3, wv.BF16, C.byref(n)) == wv.OK
    assert n.value == 9 * 192 * 32
    assert L.wanvae_packed_conv2d_weight_elems(192, 96, wv.F32, C.byref(n)) == wv.ERR_DTYPE
    assert L.wanvae_pack_conv2d_weights(p, C.c_void_p((1 << 24) + 4096), 64, 64, wv.BF16, None) == wv.ERR_ALIAS
    assert L.wanvae_pack_conv2d_weights(None, q, 64, 64, wv.BF16, None) == wv.ERR_NULL


def test_forward_noalloc_validation():
    """The allocation-free forward checks its arguments on the host, and
    rejects a block whose workspace exceeds the library's own 64 MiB array
    before it looks up or touches any device memory."""
    L = wv.lib()
    p = _params()
    x, y = C.c_void_p(1 << 34), C.c_void_p(1 << 35)
    big = wv.Dims(1, 21, 90, 160)
    assert L.wanvae_resblock_forward_noalloc(C.byref(p), x, y, C.byref(big), None) == wv.ERR_WORKSPACE
    assert "scratch" in wv.last_error()
    assert L.wanvae_resblock_forward_noalloc(None, x, y, C.byref(big), None) == wv.ERR_NULL
    p2 = _params(shortcut=False)
    assert L.wanvae_resblock_forward_noalloc(C.byref(p2), x, y, C.byref(big), None) == wv.ERR_SHAPE
    empty = wv.Dims(1, 0, 8, 32)
    assert L.wanvae_resblock_forward_noalloc(C.byref(p), None, None, C.byref(empty), None) == wv.OK


def test_stream_cache_io_validation():
    L = wv.lib()
    p, q = C.c_void_p(1 << 24), C.c_void_p(1 << 34)
    d = _dims(1, 1, 4, 8)
    for f in (L.wanvae_stream_cache_export, L.wanvae_stream_cache_import):
        assert f(p, q, C.byref(d), 24, wv.BF16, None) == wv.ERR_SHAPE     # bf16 needs C % 16
        assert f(p, q, C.byref(d), 0, wv.F32, None) == wv.ERR_SHAPE
        assert f(p, q, C.byref(d), 64, 9, None) == wv.ERR_DTYPE
        assert f(None, q, C.byref(d), 64, wv.BF16, None) == wv.ERR_NULL
        assert f(p, q, None, 64, wv.BF16, None) == wv.ERR_NULL
        assert f(p, C.c_void_p((1 << 24) + 64), C.byref(d), 64, wv.BF16, None) == wv.ERR_ALIAS
        assert f(p, C.c_void_p((1 << 34) + 8), C.byref(d), 64, wv.BF16, None) == wv.ERR_SHAPE
        empty = _dims(0, 1, 4, 8)
        assert f(None, None, C.byref(empty), 64, wv.BF16, None) == wv.OK


def test_upsample3d_validation():
    L = wv.lib()
    p, q = C.c_void_p(1 << 24), C.c_void_p(1 << 34)
    d = _dims()
    up = L.wanvae_upsample3d_conv
    assert up(p, p, None, q, C.byref(d), 64, 32, wv.F32, None) == wv.ERR_DTYPE     # bf16 only
    assert up(p, p, None, q, C.byref(d), 24, 32, wv.BF16, None) == wv.ERR_SHAPE    # cin % 16
    assert up(None, p, None, q, C.byref(d), 64, 32, wv.BF16, None) == wv.ERR_NULL
    # y (2t - 1 frames of 2h x 2w) may not overlap x
    assert up(p, q, None, C.c_void_p((1 << 24) + 1024), C.byref(d), 64, 32, wv.BF16, None) == wv.ERR_ALIAS
    empty = _dims(1, 0, 3, 4)
    assert up(None, None, None, None, C.byref(empty), 64, 32, wv.BF16, None) == wv.OK


def test_rmsnorm_silu_conv_out_validation():
    L = wv.lib()
    p, g, q = C.c_void_p(1 << 24), C.c_void_p(1 << 30), C.c_void_p(1 << 34)
    d = _dims()
    f = L.wanvae_rmsnorm_silu_conv_out
    assert f(p, None, g, None, 1e-6, p, None, q, C.byref(d), 96, 3, wv.F32, None) == wv.ERR_DTYPE  # bf16 only
    assert f(p, None, g, None, 1e-6, p, None, q, C.byref(d), 112, 3, wv.BF16, None) == wv.ERR_SHAPE  # cin <= 96
    assert f(p, None, g, None, 1e-6, p, None, q, C.byref(d), 24, 3, wv.BF16, None) == wv.ERR_SHAPE   # cin % 16
    assert f(p, None, g, None, 1e-6, p, None, q, C.byref(d), 96, 4, wv.BF16, None) == wv.ERR_SHAPE   # cout <= 3
    assert f(p, None, g, None, -1.0, p, None, q, C.byref(d), 96, 3, wv.BF16, None) == wv.ERR_SHAPE   # eps >= 0
    assert f(p, None, None, None, 1e-6, p, None, q, C.byref(d), 96, 3, wv.BF16, None) == wv.ERR_NULL  # gamma
    assert f(p, None, g, None, 1e-6, p, None, C.c_void_p((1 << 24) + 1024), C.byref(d), 96, 3, wv.BF16,
             None) == wv.ERR_ALIAS                                                                  # y overlaps x
    empty = _dims(1, 0, 3, 4)
    assert f(None, None, None, None, 1e-6, None, None, None, C.byref(empty), 96, 3, wv.BF16, None) == wv.OK
