"""CPU oracle for the Wan 2.2 VAE-decoder ResidualBlock (test infrastructure).

Thin ctypes wrapper around ``oracle.c``.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package; the product path
(``causal_convolution_amd``) never does.  Arrays are numpy float32, C-contiguous:

* activations channels-last ``[N, T, H, W, C]``;
* 3x3x3 conv weights in the pages' order ``[C_out, C_in, kD, kH, kW]``;
* 1x1x1 shortcut weights ``[C_out, C_in]``.

Every function and the readings it rests on are documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# the mutation test points this at deliberately broken builds of oracle.c
_LIB_PATH = os.environ.get("WANVAE_ORACLE_LIB", _DEFAULT_LIB)

EPS = 1e-12

_f32p = C.POINTER(C.c_float)
_i64 = C.c_int64


class _Block(C.Structure):
    _fields_ = [
        ("cin", C.c_int), ("cout", C.c_int), ("eps", C.c_double),
        ("gamma1", _f32p), ("beta1", _f32p), ("wa", _f32p), ("ba", _f32p),
        ("gamma2", _f32p), ("beta2", _f32p), ("wb", _f32p), ("bb", _f32p),
        ("ws", _f32p), ("bs", _f32p),
    ]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C99 + OpenMP).

    ``-ffp-contract=off`` keeps every multiply and add separately rounded and
    no fast-math flag is used, so the fp64 sums run in source order.
    """
    return build_to(_DEFAULT_LIB, _SRC, verbose)


def build_to(out_path: str, src: str = _SRC, verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", out_path + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(out_path + ".tmp", out_path)
    return out_path


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) and _LIB_PATH == _DEFAULT_LIB:
            build()
        L = C.CDLL(_LIB_PATH)
        L.oracle_silu.restype = C.c_double
        L.oracle_silu.argtypes = [C.c_double]
        L.oracle_num_threads.restype = C.c_int
        L.oracle_norm_silu.argtypes = [_f32p, _f32p, _i64, C.c_int, _f32p, _f32p, C.c_double]
        L.oracle_rms_norm.argtypes = [_f32p, _f32p, _i64, C.c_int, _f32p, _f32p, C.c_double]
        L.oracle_causal_conv3d.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p,
                                           _i64, _i64, _i64, _i64, C.c_int, C.c_int]
        L.oracle_shortcut.argtypes = [C.POINTER(_Block), _f32p, _f32p, _i64, _i64, _i64, _i64]
        L.oracle_resblock_full.argtypes = [C.POINTER(_Block), _f32p, _f32p, _i64, _i64, _i64, _i64]
        L.oracle_resblock_stream_step.argtypes = [C.POINTER(_Block), _f32p, _f32p,
                                                  _i64, _i64, _i64, _i64, _f32p, _f32p]
        L.oracle_resblock_stream.argtypes = [C.POINTER(_Block), _f32p, _f32p,
                                             _i64, _i64, _i64, _i64, _i64]
        L.oracle_resblock_window.argtypes = [C.POINTER(_Block), _f32p] + [_i64] * 16 + [_f32p]
        L.oracle_attention_frame.argtypes = [_f32p, _i64, C.c_int, _f32p, _f32p, C.c_double,
                                             _f32p, _f32p, _f32p, _f32p, C.POINTER(C.c_int64),
                                             _i64, _f32p]
        L.oracle_attention_frame.restype = None
        L.oracle_upsample2d_conv.argtypes = [_f32p, _i64, _i64, _i64, C.c_int, C.c_int, _f32p, _f32p,
                                             _i64, _i64, _f32p]
        L.oracle_upsample2d_conv.restype = None
        L.oracle_upsample3d_conv.argtypes = [_f32p, _i64, _i64, _i64, _i64, C.c_int, C.c_int, _f32p, _f32p,
                                             _f32p]
        L.oracle_upsample3d_conv.restype = None
        for f in ("oracle_norm_silu", "oracle_rms_norm", "oracle_causal_conv3d", "oracle_shortcut",
                  "oracle_resblock_full", "oracle_resblock_stream_step",
                  "oracle_resblock_stream", "oracle_resblock_window"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_f32p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def silu(u: float) -> float:
    return lib().oracle_silu(float(u))


def norm_silu(x, gamma, beta=None, eps: float = EPS):
    """silu(RMS_norm over the last axis) of float32 x (any leading shape)."""
    x = _f32(x)
    C_ = x.shape[-1]
    gamma = _f32(gamma)
    beta = None if beta is None else _f32(beta)
    assert gamma.shape == (C_,) and (beta is None or beta.shape == (C_,))
    y = np.empty_like(x)
    lib().oracle_norm_silu(_ptr(x), _ptr(y), x.size // C_ if C_ else 0, C_, _ptr(gamma),
                           _ptr(beta), float(eps))
    return y


def rms_norm(x, gamma, beta=None, eps: float = EPS):
    """RMS_norm over the last axis (no activation), rounded to float32."""
    x = _f32(x)
    C_ = x.shape[-1]
    gamma = _f32(gamma)
    beta = None if beta is None else _f32(beta)
    assert gamma.shape == (C_,) and (beta is None or beta.shape == (C_,))
    y = np.empty_like(x)
    lib().oracle_rms_norm(_ptr(x), _ptr(y), x.size // C_ if C_ else 0, C_, _ptr(gamma),
                          _ptr(beta), float(eps))
    return y


def causal_conv3d(x, w, bias=None, cache=None):
    """Causal 3x3x3 conv: x [N,T,H,W,Cin], w [Cout,Cin,3,3,3] -> [N,T,H,W,Cout]."""
    x = _f32(x)
    w = _f32(w)
    N, T, H, W, Cin = x.shape
    Cout = w.shape[0]
    assert w.shape == (Cout, Cin, 3, 3, 3)
    bias = None if bias is None else _f32(bias)
    if cache is not None:
        cache = _f32(cache)
        assert cache.shape == (N, 2, H, W, Cin)
    y = np.empty((N, T, H, W, Cout), np.float32)
    lib().oracle_causal_conv3d(_ptr(x), _ptr(cache), _ptr(w), _ptr(bias), _ptr(y),
                               N, T, H, W, Cin, Cout)
    return y


class Block:
    """ResidualBlock parameters as float32 numpy arrays (pages' weight order)."""

    def __init__(self, gamma1, beta1, wa, ba, gamma2, beta2, wb, bb, ws=None, bs=None,
                 eps: float = EPS):
        self.gamma1, self.beta1 = _f32(gamma1), None if beta1 is None else _f32(beta1)
        self.wa, self.ba = _f32(wa), None if ba is None else _f32(ba)
        self.gamma2, self.beta2 = _f32(gamma2), None if beta2 is None else _f32(beta2)
        self.wb, self.bb = _f32(wb), None if bb is None else _f32(bb)
        self.ws = None if ws is None else _f32(ws)
        self.bs = None if bs is None else _f32(bs)
        self.eps = float(eps)
        self.cout, self.cin = self.wa.shape[0], self.wa.shape[1]
        assert self.wa.shape == (self.cout, self.cin, 3, 3, 3)
        assert self.wb.shape == (self.cout, self.cout, 3, 3, 3)
        if self.ws is None:
            assert self.cin == self.cout, "identity shortcut needs in_dim == out_dim"
        else:
            assert self.ws.shape == (self.cout, self.cin)

    def _c(self):
        return _Block(self.cin, self.cout, self.eps, _ptr(self.gamma1), _ptr(self.beta1),
                      _ptr(self.wa), _ptr(self.ba), _ptr(self.gamma2), _ptr(self.beta2),
                      _ptr(self.wb), _ptr(self.bb), _ptr(self.ws), _ptr(self.bs))


def shortcut(blk: Block, x):
    x = _f32(x)
    N, T, H, W, _ = x.shape
    y = np.empty((N, T, H, W, blk.cout), np.float32)
    cb = blk._c()
    lib().oracle_shortcut(C.byref(cb), _ptr(x), _ptr(y), N, T, H, W)
    return y


def pointwise_conv(x, w, bias=None):
    """1x1x1 conv over channels-last positions: x [..., Cin], w [Cout, Cin]
    -> [..., Cout], y = bias + sum_ci w[co, ci] x[..., ci] (fp64 sum, one
    rounding).  The decoder's post_quant_conv is a CausalConv3d of kernel 1
    ("Sharding of WAN 2.2 VAE", decoder module tree); kernel 1 has no causal
    pad.  Same routine as the block's 1x1x1 shortcut."""
    x = _f32(x)
    w = _f32(w)
    cout, cin = w.shape
    assert x.shape[-1] == cin
    bias = None if bias is None else _f32(bias)
    rows = x.reshape(1, 1, 1, -1, cin)
    y = np.empty(rows.shape[:-1] + (cout,), np.float32)
    cb = _Block(cin, cout, 0.0, None, None, None, None, None, None, None, None, _ptr(w), _ptr(bias))
    lib().oracle_shortcut(C.byref(cb), _ptr(np.ascontiguousarray(rows)), _ptr(y), 1, 1, 1, rows.shape[3])
    return y.reshape(x.shape[:-1] + (cout,))


def attention_block(x, gamma, beta, wqkv, bqkv, wo, bo, eps: float = EPS, frame=None,
                    queries=None):
    """Decoder mid-block attention (readings in oracle.c, oracle_attention_frame).

    x [N,T,H,W,C]; wqkv [3C,C], bqkv [3C] (q, k, v rows in that order); wo [C,C],
    bo [C].  Returns y [N,T,H,W,C] for every frame, or, with frame=(n, t) and
    queries (flat h*W+w indices of that frame), y at those positions [nq, C]."""
    x = _f32(x)
    N, T, H, W, C_ = x.shape
    HW = H * W
    g, wqkv, wo = _f32(gamma), _f32(wqkv), _f32(wo)
    b = None if beta is None else _f32(beta)
    bq = None if bqkv is None else _f32(bqkv)
    bo_ = None if bo is None else _f32(bo)
    assert wqkv.shape == (3 * C_, C_) and wo.shape == (C_, C_)

    def run(frame_x, qidx):
        fx = np.ascontiguousarray(frame_x.reshape(HW, C_))
        nq = HW if qidx is None else len(qidx)
        y = np.empty((nq, C_), np.float32)
        qi = None if qidx is None else np.ascontiguousarray(qidx, dtype=np.int64)
        lib().oracle_attention_frame(
            _ptr(fx), HW, C_, _ptr(g), _ptr(b), float(eps), _ptr(wqkv), _ptr(bq), _ptr(wo),
            _ptr(bo_), None if qi is None else qi.ctypes.data_as(C.POINTER(C.c_int64)), nq,
            _ptr(y))
        return y

    if frame is not None:
        n, t = frame
        return run(x[n, t], queries)
    out = np.empty_like(x)
    for n in range(N):
        for t in range(T):
            out[n, t] = run(x[n, t], None).reshape(H, W, C_)
    return out


def resblock_full(blk: Block, x):
    x = _f32(x)
    N, T, H, W, Cin = x.shape
    assert Cin == blk.cin
    y = np.empty((N, T, H, W, blk.cout), np.float32)
    cb = blk._c()
    lib().oracle_resblock_full(C.byref(cb), _ptr(x), _ptr(y), N, T, H, W)
    return y


def resblock_stream_step(blk: Block, x_chunk, cache_a, cache_b):
    """One streaming step; cache_a/cache_b (float32, C-contiguous) update in place."""
    x_chunk = _f32(x_chunk)
    N, Tc, H, W, Cin = x_chunk.shape
    assert cache_a.shape == (N, 2, H, W, blk.cin) and cache_a.dtype == np.float32
    assert cache_b.shape == (N, 2, H, W, blk.cout) and cache_b.dtype == np.float32
    assert cache_a.flags["C_CONTIGUOUS"] and cache_b.flags["C_CONTIGUOUS"]
    y = np.empty((N, Tc, H, W, blk.cout), np.float32)
    cb = blk._c()
    lib().oracle_resblock_stream_step(C.byref(cb), _ptr(x_chunk), _ptr(y), N, Tc, H, W,
                                      _ptr(cache_a), _ptr(cache_b))
    return y


def resblock_stream(blk: Block, x, t_step: int = 1):
    x = _f32(x)
    N, T, H, W, Cin = x.shape
    y = np.empty((N, T, H, W, blk.cout), np.float32)
    cb = blk._c()
    lib().oracle_resblock_stream(C.byref(cb), _ptr(x), _ptr(y), N, T, H, W, int(t_step))
    return y


def receptive_region(box, dims):
    """x region (t0, t1, h0, h1, w0, w1) that an output box of the block depends on."""
    T, H, W = dims
    t0, t1, h0, h1, w0, w1 = box
    return (max(t0 - 4, 0), t1, max(h0 - 2, 0), min(h1 + 2, H), max(w0 - 2, 0), min(w1 + 2, W))


def resblock_window(blk: Block, x_region, region, dims, box):
    """Block output on ``box`` = (t0,t1,h0,h1,w0,w1) of a full tensor of extent
    ``dims`` = (T,H,W), from ``x_region`` = x[:, rt0:rt1, rh0:rh1, rw0:rw1]
    where ``region`` must be ``receptive_region(box, dims)``."""
    x_region = _f32(x_region)
    T, H, W = dims
    rt0, rt1, rh0, rh1, rw0, rw1 = region
    assert tuple(region) == receptive_region(box, dims)
    N = x_region.shape[0]
    assert x_region.shape == (N, rt1 - rt0, rh1 - rh0, rw1 - rw0, blk.cin)
    t0, t1, h0, h1, w0, w1 = box
    assert 0 <= t0 < t1 <= T and 0 <= h0 < h1 <= H and 0 <= w0 < w1 <= W
    y = np.empty((N, t1 - t0, h1 - h0, w1 - w0, blk.cout), np.float32)
    cb = blk._c()
    lib().oracle_resblock_window(C.byref(cb), _ptr(x_region), N, T, H, W, rt0, rh0, rw0,
                                 rt1 - rt0, rh1 - rh0, rw1 - rw0, t0, t1, h0, h1, w0, w1,
                                 _ptr(y))
    return y


def upsample2d_conv(x, w, bias=None, frames=None, rows=None):
    """The decoder's spatial upsampler (readings in oracle.c,
    oracle_upsample2d_conv): nearest-neighbour x2 in H and W, then a 3x3 conv
    with zero padding 1, frame by frame.

    x [N,T,H,W,Cin]; w [Cout,Cin,3,3]; bias [Cout] or None.  Returns y
    [N,T,2H,2W,Cout], or with frames (a list of (n, t)) and rows (r0, r1) only
    those output rows of those frames, [len(frames), r1 - r0, 2W, Cout]."""
    x = _f32(x)
    w = _f32(w)
    N, T, H, W, cin = x.shape
    cout = w.shape[0]
    assert w.shape == (cout, cin, 3, 3)
    bias = None if bias is None else _f32(bias)
    r0, r1 = (0, 2 * H) if rows is None else rows
    assert 0 <= r0 <= r1 <= 2 * H
    if frames is None:
        xs = x.reshape(N * T, H, W, cin)
    else:
        xs = np.ascontiguousarray(np.stack([x[n, t] for (n, t) in frames]))
    nf = xs.shape[0]
    y = np.empty((nf, r1 - r0, 2 * W, cout), np.float32)
    lib().oracle_upsample2d_conv(_ptr(xs), nf, H, W, cin, cout, _ptr(w), _ptr(bias), r0, r1, _ptr(y))
    return y.reshape(N, T, r1 - r0, 2 * W, cout) if frames is None else y


def upsample3d_conv(x, w, bias=None):
    """The decoder's upsample3d (readings in oracle.c, oracle_upsample3d_conv):
    T frames to 2T - 1, output frame t' being input frame (t' + 1) // 2, then
    each frame through upsample2d_conv.  x [N,T,H,W,Cin] (T >= 1); w
    [Cout,Cin,3,3]; bias [Cout] or None.  Returns [N,2T-1,2H,2W,Cout]."""
    x = _f32(x)
    w = _f32(w)
    N, T, H, W, cin = x.shape
    assert T >= 1
    cout = w.shape[0]
    assert w.shape == (cout, cin, 3, 3)
    bias = None if bias is None else _f32(bias)
    y = np.empty((N, 2 * T - 1, 2 * H, 2 * W, cout), np.float32)
    lib().oracle_upsample3d_conv(_ptr(x), N, T, H, W, cin, cout, _ptr(w), _ptr(bias), _ptr(y))
    return y
