"""Wan 2.2 VAE-decoder ResidualBlock on MI355X: Python binding of libwanvae.so.

Argument marshalling only: every entry point takes torch tensors that live on
the GPU, checks their dtype / shape / contiguity, and passes raw device
pointers plus torch's current HIP stream to the C ABI declared in
``include/wanvae.h``.  All computation happens in the library's HIP kernels;
there is no other implementation and no fallback: if ``libwanvae.so`` is not
built, importing the binding's functions raises.

Layouts: activations are channels-last ``[n, t, h, w, C]``; 3x3x3 conv
weights enter in the PyTorch Conv3d layout ``[C_out, C_in, 3, 3, 3]`` and are
packed once on the GPU (``pack_conv3d_weights``) into the order the conv
kernels stream; the shortcut weight is ``[C_out, C_in]``.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwanvae.so")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP = range(7)
F32, BF16 = 0, 1
(KERNEL_NORM, KERNEL_CONV_BF16, KERNEL_CONV_F32, KERNEL_ROLL, KERNEL_POINTWISE, KERNEL_GEMM,
 KERNEL_TRANSPOSE, KERNEL_ATTENTION, KERNEL_UPSAMPLE, KERNEL_COPY) = range(10)
EPS = 1e-12


class WanVaeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"wanvae status {status}: {msg}")
        self.status = status


class Dims(C.Structure):
    _fields_ = [("n", C.c_int64), ("t", C.c_int64), ("h", C.c_int64), ("w", C.c_int64)]


class ResblockParamsC(C.Structure):
    _fields_ = [
        ("in_dim", C.c_int32), ("out_dim", C.c_int32), ("dtype", C.c_int32), ("eps", C.c_float),
        ("gamma1", C.c_void_p), ("beta1", C.c_void_p), ("w_a", C.c_void_p), ("b_a", C.c_void_p),
        ("gamma2", C.c_void_p), ("beta2", C.c_void_p), ("w_b", C.c_void_p), ("b_b", C.c_void_p),
        ("w_sc", C.c_void_p), ("b_sc", C.c_void_p),
    ]


EXPORTS = {
    "wanvae_rmsnorm_silu": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p,
                                      C.c_void_p, C.c_float, C.c_int32, C.c_void_p]),
    "wanvae_pack_conv3d_weights": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                             C.c_void_p]),
    "wanvae_causal_conv3d": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.POINTER(Dims), C.c_int32, C.c_int32, C.c_int32,
                                       C.c_void_p]),
    "wanvae_rmsnorm_silu_conv_out": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_float,
                                               C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(Dims),
                                               C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "wanvae_resblock_workspace_size": (C.c_int, [C.POINTER(ResblockParamsC), C.POINTER(Dims),
                                                 C.POINTER(C.c_size_t)]),
    "wanvae_resblock_forward": (C.c_int, [C.POINTER(ResblockParamsC), C.c_void_p, C.c_void_p,
                                          C.POINTER(Dims), C.c_void_p, C.c_size_t, C.c_void_p]),
    "wanvae_resblock_stream_step": (C.c_int, [C.POINTER(ResblockParamsC), C.c_void_p, C.c_void_p,
                                              C.POINTER(Dims), C.c_void_p, C.c_void_p,
                                              C.c_void_p, C.c_size_t, C.c_void_p]),
    "wanvae_packed_conv3d_weight_elems": (C.c_int, [C.c_int32, C.c_int32, C.c_int32,
                                                    C.POINTER(C.c_int64)]),
    "wanvae_pointwise_conv": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                        C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "wanvae_attention_workspace_size": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(C.c_size_t)]),
    "wanvae_attention_block": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_size_t, C.c_void_p]),
    "wanvae_upsample2d_conv": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(Dims),
                                         C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "wanvae_upsample3d_conv": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(Dims),
                                         C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "wanvae_pack_conv2d_weights": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                             C.c_void_p]),
    "wanvae_packed_conv2d_weight_elems": (C.c_int, [C.c_int32, C.c_int32, C.c_int32,
                                                    C.POINTER(C.c_int64)]),
    "wanvae_resblock_forward_noalloc": (C.c_int, [C.POINTER(ResblockParamsC), C.c_void_p, C.c_void_p,
                                                  C.POINTER(Dims), C.c_void_p]),
    "wanvae_wait_giveups": (C.c_int, [C.POINTER(C.c_uint64)]),
    "wanvae_wait_giveups_reset": (C.c_int, []),
    "wanvae_set_wait_bound": (C.c_int, [C.c_int32]),
    "wanvae_stream_cache_export": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(Dims), C.c_int32, C.c_int32,
                                             C.c_void_p]),
    "wanvae_stream_cache_import": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(Dims), C.c_int32, C.c_int32,
                                             C.c_void_p]),
    "wanvae_stream_copy": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p]),
    "wanvae_last_error": (C.c_char_p, []),
    "wanvae_timing_enable": (C.c_int, [C.c_int]),
    "wanvae_timing_reset": (C.c_int, []),
    "wanvae_timing_read": (C.c_int, [C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_double)]),
}

_lib = None


def lib():
    """The loaded libwanvae.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m causal_convolution_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().wanvae_last_error().decode()


def _check(status: int):
    if status != OK:
        raise WanVaeError(status, last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


# --------------------------------------------------------------------------- single ops
def rmsnorm_silu(x, gamma, beta=None, eps: float = EPS, out=None, stream=None):
    """y = silu(RMS_norm over the last axis of x) (``wanvae_rmsnorm_silu``)."""
    torch = _torch()
    Cc = x.shape[-1]
    _dev(x, "x")
    _dev(gamma, "gamma", torch.float32, (Cc,))
    _dev(beta, "beta", torch.float32, (Cc,))
    y = torch.empty_like(x) if out is None else out
    _dev(y, "out", x.dtype, x.shape)
    rows = x.numel() // Cc if Cc else 0
    _check(lib().wanvae_rmsnorm_silu(_ptr(x), _ptr(y), rows, Cc, _ptr(gamma), _ptr(beta),
                                     float(eps), _dtype_code(x), _stream(stream)))
    return y


class PackedWeight:
    """A 3x3x3 conv weight packed by ``wanvae_pack_conv3d_weights``: ``data`` is
    a flat device tensor of ``packed_conv3d_weight_elems(cin, cout, dtype)``
    elements (27 * cin * cout, with cout rounded up to 32 for bf16)."""

    def __init__(self, data, cin: int, cout: int):
        self.data, self.cin, self.cout = data, int(cin), int(cout)

    @property
    def dtype(self):
        return self.data.dtype


def pack_conv3d_weights(w, stream=None) -> PackedWeight:
    """Pack a conv weight [C_out, C_in, 3, 3, 3] (PyTorch Conv3d layout, on the
    GPU, bf16 or fp32) for the conv kernels (``wanvae_pack_conv3d_weights``)."""
    torch = _torch()
    if w.dim() != 5 or tuple(w.shape[2:]) != (3, 3, 3):
        raise ValueError(f"w must be [C_out, C_in, 3, 3, 3], got {tuple(w.shape)}")
    _dev(w, "w")
    cout, cin = int(w.shape[0]), int(w.shape[1])
    out = torch.empty(packed_conv3d_weight_elems(cin, cout, _dtype_code(w)), dtype=w.dtype,
                      device=w.device)
    _check(lib().wanvae_pack_conv3d_weights(_ptr(w), _ptr(out), cin, cout, _dtype_code(w),
                                            _stream(stream)))
    return PackedWeight(out, cin, cout)


def packed_conv3d_weight_elems(cin: int, cout: int, dtype_code: int) -> int:
    """Elements of a packed conv weight (``wanvae_packed_conv3d_weight_elems``)."""
    n = C.c_int64(0)
    _check(lib().wanvae_packed_conv3d_weight_elems(int(cin), int(cout), int(dtype_code), C.byref(n)))
    return n.value


def _packed(w, name, dtype, cin, cout):
    if not isinstance(w, PackedWeight):
        raise TypeError(f"{name} must be a PackedWeight (see pack_conv3d_weights)")
    if (w.cin, w.cout) != (cin, cout):
        raise ValueError(f"{name} is {w.cin}->{w.cout}, expected {cin}->{cout}")
    _dev(w.data, name, dtype, (packed_conv3d_weight_elems(cin, cout, _dtype_code(w.data)),))


def pointwise_conv(x, w, bias=None, out=None, stream=None):
    """Pointwise (1x1x1) conv (``wanvae_pointwise_conv``): x [..., Cin]
    channels-last, w [Cout, Cin] of x's dtype, bias [Cout] fp32 or None ->
    [..., Cout]."""
    torch = _torch()
    cin = int(x.shape[-1])
    cout = int(w.shape[0])
    _dev(x, "x")
    _dev(w, "w", x.dtype, (cout, cin))
    _dev(bias, "bias", torch.float32, (cout,))
    y = torch.empty(tuple(x.shape[:-1]) + (cout,), dtype=x.dtype, device=x.device) if out is None else out
    _dev(y, "out", x.dtype, tuple(x.shape[:-1]) + (cout,))
    rows = x.numel() // cin if cin else 0
    _check(lib().wanvae_pointwise_conv(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), rows, cin, cout,
                                       _dtype_code(x), _stream(stream)))
    return y


def causal_conv3d(x, w, bias=None, cache=None, out=None, stream=None):
    """Causal 3x3x3 conv (``wanvae_causal_conv3d``): x [n,t,h,w,Cin], w a
    PackedWeight (Cin -> Cout), cache [n,2,h,w,Cin] or None -> [n,t,h,w,Cout]."""
    torch = _torch()
    n, t, h, wd, cin = x.shape
    cout = w.cout
    _dev(x, "x")
    _packed(w, "w", x.dtype, cin, cout)
    _dev(bias, "bias", torch.float32, (cout,))
    _dev(cache, "cache", x.dtype, (n, 2, h, wd, cin))
    y = torch.empty((n, t, h, wd, cout), dtype=x.dtype, device=x.device) if out is None else out
    _dev(y, "out", x.dtype, (n, t, h, wd, cout))
    d = Dims(n, t, h, wd)
    _check(lib().wanvae_causal_conv3d(_ptr(x), _ptr(cache), _ptr(w.data), _ptr(bias), _ptr(y),
                                      C.byref(d), cin, cout, _dtype_code(x), _stream(stream)))
    return y


def rmsnorm_silu_conv_out(x, gamma, beta, eps, w, bias=None, cache=None, out=None, stream=None):
    """The decoder's norm_out -> SiLU -> conv_out in one pass
    (``wanvae_rmsnorm_silu_conv_out``, bf16): x [n,t,h,w,Cin] the norm's
    input, gamma/beta [Cin] fp32, w a PackedWeight (Cin -> Cout <= 3), cache
    [n,2,h,w,Cin] of the norm's input or None -> [n,t,h,w,Cout]."""
    torch = _torch()
    n, t, h, wd, cin = x.shape
    cout = w.cout
    _dev(x, "x", torch.bfloat16)
    _packed(w, "w", x.dtype, cin, cout)
    _dev(gamma, "gamma", torch.float32, (cin,))
    _dev(beta, "beta", torch.float32, (cin,))
    _dev(bias, "bias", torch.float32, (cout,))
    _dev(cache, "cache", x.dtype, (n, 2, h, wd, cin))
    y = torch.empty((n, t, h, wd, cout), dtype=x.dtype, device=x.device) if out is None else out
    _dev(y, "out", x.dtype, (n, t, h, wd, cout))
    d = Dims(n, t, h, wd)
    _check(lib().wanvae_rmsnorm_silu_conv_out(_ptr(x), _ptr(cache), _ptr(gamma), _ptr(beta), float(eps),
                                              _ptr(w.data), _ptr(bias), _ptr(y), C.byref(d), cin, cout,
                                              _dtype_code(x), _stream(stream)))
    return y


# --------------------------------------------------------------------------- upsampler
class PackedWeight2d:
    """A 3x3 conv weight packed by ``wanvae_pack_conv2d_weights`` (bf16):
    ``data`` holds ``packed_conv2d_weight_elems(cin, cout)`` elements."""

    def __init__(self, data, cin: int, cout: int):
        self.data, self.cin, self.cout = data, int(cin), int(cout)


def packed_conv2d_weight_elems(cin: int, cout: int) -> int:
    """Elements of a packed 2D conv weight (``wanvae_packed_conv2d_weight_elems``)."""
    n = C.c_int64(0)
    _check(lib().wanvae_packed_conv2d_weight_elems(int(cin), int(cout), BF16, C.byref(n)))
    return n.value


def pack_conv2d_weights(w, stream=None) -> PackedWeight2d:
    """Pack a 3x3 conv weight [C_out, C_in, 3, 3] (bf16, on the GPU) for
    ``upsample2d_conv``."""
    torch = _torch()
    if w.dim() != 4 or tuple(w.shape[2:]) != (3, 3):
        raise ValueError(f"w must be [C_out, C_in, 3, 3], got {tuple(w.shape)}")
    _dev(w, "w", torch.bfloat16)
    cout, cin = int(w.shape[0]), int(w.shape[1])
    out = torch.empty(packed_conv2d_weight_elems(cin, cout), dtype=w.dtype, device=w.device)
    _check(lib().wanvae_pack_conv2d_weights(_ptr(w), _ptr(out), cin, cout, BF16, _stream(stream)))
    return PackedWeight2d(out, cin, cout)


def upsample2d_conv(x, w, bias=None, out=None, stream=None):
    """The decoder's spatial upsampler (``wanvae_upsample2d_conv``): x
    [n,t,h,w,Cin] bf16, w a PackedWeight2d (Cin -> Cout), bias [Cout] fp32 or
    None -> [n,t,2h,2w,Cout]: nearest-neighbour x2, then the 3x3 conv."""
    torch = _torch()
    n, t, h, wd, cin = x.shape
    if not isinstance(w, PackedWeight2d):
        raise TypeError("w must be a PackedWeight2d (see pack_conv2d_weights)")
    if w.cin != cin:
        raise ValueError(f"w is {w.cin}->{w.cout}, x has {cin} channels")
    cout = w.cout
    _dev(x, "x", torch.bfloat16)
    _dev(w.data, "w", torch.bfloat16, (packed_conv2d_weight_elems(cin, cout),))
    _dev(bias, "bias", torch.float32, (cout,))
    shape = (n, t, 2 * h, 2 * wd, cout)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    _dev(y, "out", x.dtype, shape)
    d = Dims(n, t, h, wd)
    _check(lib().wanvae_upsample2d_conv(_ptr(x), _ptr(w.data), _ptr(bias), _ptr(y), C.byref(d), cin, cout,
                                        BF16, _stream(stream)))
    return y


def upsample3d_conv(x, w, bias=None, out=None, stream=None):
    """The decoder's upsample3d (``wanvae_upsample3d_conv``): x [n,t,h,w,Cin]
    bf16, w a PackedWeight2d (Cin -> Cout), bias [Cout] fp32 or None ->
    [n,2t-1,2h,2w,Cout]: output frame t' is input frame (t'+1)//2, doubled
    in H and W by nearest neighbour, then the 3x3 conv."""
    torch = _torch()
    n, t, h, wd, cin = x.shape
    if not isinstance(w, PackedWeight2d):
        raise TypeError("w must be a PackedWeight2d (see pack_conv2d_weights)")
    if w.cin != cin:
        raise ValueError(f"w is {w.cin}->{w.cout}, x has {cin} channels")
    cout = w.cout
    _dev(x, "x", torch.bfloat16)
    _dev(w.data, "w", torch.bfloat16, (packed_conv2d_weight_elems(cin, cout),))
    _dev(bias, "bias", torch.float32, (cout,))
    shape = (n, max(2 * t - 1, 0), 2 * h, 2 * wd, cout)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    _dev(y, "out", x.dtype, shape)
    d = Dims(n, t, h, wd)
    _check(lib().wanvae_upsample3d_conv(_ptr(x), _ptr(w.data), _ptr(bias), _ptr(y), C.byref(d), cin, cout,
                                        BF16, _stream(stream)))
    return y


# --------------------------------------------------------------------------- block
class ResBlock:
    """Device-resident parameters of one ResidualBlock.

    ``w_a`` and ``w_b`` are PackedWeights.  ``from_host`` takes float32 numpy
    arrays with conv weights in the pages' order [C_out, C_in, kD, kH, kW],
    uploads them in the block's dtype and packs them on the GPU, once, at setup.
    """

    def __init__(self, in_dim, out_dim, dtype, gamma1, beta1, w_a, b_a, gamma2, beta2, w_b, b_b,
                 w_sc=None, b_sc=None, eps: float = EPS):
        torch = _torch()
        self.in_dim, self.out_dim, self.eps = int(in_dim), int(out_dim), float(eps)
        self.dtype = dtype
        self.tensors = dict(gamma1=gamma1, beta1=beta1, w_a=w_a, b_a=b_a, gamma2=gamma2,
                            beta2=beta2, w_b=w_b, b_b=b_b, w_sc=w_sc, b_sc=b_sc)
        ci, co = self.in_dim, self.out_dim
        shapes = dict(gamma1=(ci,), beta1=(ci,), b_a=(co,), gamma2=(co,), beta2=(co,), b_b=(co,),
                      b_sc=(co,))
        for k, shp in shapes.items():
            _dev(self.tensors[k], k, torch.float32, shp)
        _packed(w_a, "w_a", dtype, ci, co)
        _packed(w_b, "w_b", dtype, co, co)
        _dev(w_sc, "w_sc", dtype, (co, ci))
        self.c = ResblockParamsC(ci, co, BF16 if dtype == torch.bfloat16 else F32, self.eps,
                                 *[None if self.tensors[k] is None else self._ptr_of(self.tensors[k])
                                   for k in ("gamma1", "beta1", "w_a", "b_a", "gamma2", "beta2",
                                             "w_b", "b_b", "w_sc", "b_sc")])

    @staticmethod
    def _ptr_of(t):
        return t.data.data_ptr() if isinstance(t, PackedWeight) else t.data_ptr()

    @classmethod
    def from_host(cls, p: dict, dtype, device="cuda", eps: float = EPS):
        import numpy as np
        torch = _torch()

        def f32(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)

        def wt(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a, np.float32)
            return torch.from_numpy(a).to(device=device, dtype=dtype).contiguous()

        ci, co = p["wa"].shape[1], p["wa"].shape[0]
        w_a = pack_conv3d_weights(wt(p["wa"]))
        w_b = pack_conv3d_weights(wt(p["wb"]))
        torch.cuda.synchronize()
        return cls(ci, co, dtype, f32(p["gamma1"]), f32(p["beta1"]), w_a, f32(p["ba"]),
                   f32(p["gamma2"]), f32(p["beta2"]), w_b, f32(p["bb"]),
                   wt(p.get("ws")), f32(p.get("bs")), eps)

    def workspace_size(self, n, t, h, w) -> int:
        d = Dims(n, t, h, w)
        b = C.c_size_t(0)
        _check(lib().wanvae_resblock_workspace_size(C.byref(self.c), C.byref(d), C.byref(b)))
        return b.value

    def workspace(self, n, t, h, w, device="cuda"):
        torch = _torch()
        return torch.empty(max(self.workspace_size(n, t, h, w), 1), dtype=torch.uint8, device=device)

    def forward(self, x, out=None, workspace=None, stream=None):
        """Full-T block (``wanvae_resblock_forward``): x [n,t,h,w,in_dim] -> y."""
        torch = _torch()
        n, t, h, w, ci = x.shape
        _dev(x, "x", self.dtype, (n, t, h, w, self.in_dim))
        y = torch.empty((n, t, h, w, self.out_dim), dtype=x.dtype, device=x.device) if out is None else out
        _dev(y, "out", self.dtype, (n, t, h, w, self.out_dim))
        ws = self.workspace(n, t, h, w, x.device) if workspace is None else workspace
        d = Dims(n, t, h, w)
        _check(lib().wanvae_resblock_forward(C.byref(self.c), _ptr(x), _ptr(y), C.byref(d),
                                             _ptr(ws), ws.numel() * ws.element_size(),
                                             _stream(stream)))
        return y

    def forward_noalloc(self, x, out, stream=None):
        """Full-T block without a workspace (``wanvae_resblock_forward_noalloc``):
        the library's own 64 MiB device array holds the intermediates; ``out``
        must be given (nothing is allocated)."""
        n, t, h, w, ci = x.shape
        _dev(x, "x", self.dtype, (n, t, h, w, self.in_dim))
        _dev(out, "out", self.dtype, (n, t, h, w, self.out_dim))
        d = Dims(n, t, h, w)
        _check(lib().wanvae_resblock_forward_noalloc(C.byref(self.c), _ptr(x), _ptr(out), C.byref(d),
                                                     _stream(stream)))
        return out

    def new_caches(self, n, h, w, device="cuda"):
        """Zero caches for a fresh stream: flat buffers of n*2*h*w*in_dim and
        n*2*h*w*out_dim elements.  Their contents are the library's own
        conv-input frames (16-channel slices for bf16), opaque to callers:
        ``export_cache`` / ``import_cache`` read and set them channels-last."""
        torch = _torch()
        return (torch.zeros((n * 2 * h * w * self.in_dim,), dtype=self.dtype, device=device),
                torch.zeros((n * 2 * h * w * self.out_dim,), dtype=self.dtype, device=device))

    def export_cache(self, cache, n, h, w, channels, out=None, stream=None):
        """A cache's frames, channels-last (see ``export_stream_cache``);
        channels is in_dim for cache_a, out_dim for cache_b."""
        _dev(cache, "cache", self.dtype)
        return export_stream_cache(cache, n, h, w, channels, out, stream)

    def import_cache(self, frames, cache, stream=None):
        """Sets a cache from channels-last frames (see ``import_stream_cache``)."""
        _dev(cache, "cache", self.dtype)
        return import_stream_cache(frames, cache, stream)

    def stream_step(self, x_chunk, cache_a, cache_b, out=None, workspace=None, stream=None):
        """One streaming step (``wanvae_resblock_stream_step``); caches update in place."""
        torch = _torch()
        n, t, h, w, ci = x_chunk.shape
        _dev(x_chunk, "x_chunk", self.dtype, (n, t, h, w, self.in_dim))
        _dev(cache_a, "cache_a", self.dtype, (n * 2 * h * w * self.in_dim,))
        _dev(cache_b, "cache_b", self.dtype, (n * 2 * h * w * self.out_dim,))
        y = torch.empty((n, t, h, w, self.out_dim), dtype=x_chunk.dtype,
                        device=x_chunk.device) if out is None else out
        _dev(y, "out", self.dtype, (n, t, h, w, self.out_dim))
        ws = self.workspace(n, t, h, w, x_chunk.device) if workspace is None else workspace
        d = Dims(n, t, h, w)
        _check(lib().wanvae_resblock_stream_step(C.byref(self.c), _ptr(x_chunk), _ptr(y),
                                                 C.byref(d), _ptr(cache_a), _ptr(cache_b),
                                                 _ptr(ws), ws.numel() * ws.element_size(),
                                                 _stream(stream)))
        return y


def export_stream_cache(cache, n, h, w, channels, out=None, stream=None):
    """A stream cache's frames -2, -1 as a channels-last [n, 2, h, w,
    channels] tensor of the cache's dtype (``wanvae_stream_cache_export``)."""
    torch = _torch()
    _dev(cache, "cache", None, (n * 2 * h * w * channels,))
    y = torch.empty((n, 2, h, w, channels), dtype=cache.dtype, device=cache.device) if out is None else out
    _dev(y, "out", cache.dtype, (n, 2, h, w, channels))
    d = Dims(n, 2, h, w)
    _check(lib().wanvae_stream_cache_export(_ptr(cache), _ptr(y), C.byref(d), int(channels), _dtype_code(cache),
                                            _stream(stream)))
    return y


def import_stream_cache(frames, cache, stream=None):
    """Sets a stream cache from channels-last frames [n, 2, h, w, channels]
    of its dtype (``wanvae_stream_cache_import``)."""
    n, two, h, w, channels = frames.shape
    _dev(frames, "frames", cache.dtype, (n, 2, h, w, channels))
    _dev(cache, "cache", None, (n * 2 * h * w * channels,))
    d = Dims(n, 2, h, w)
    _check(lib().wanvae_stream_cache_import(_ptr(frames), _ptr(cache), C.byref(d), int(channels),
                                            _dtype_code(cache), _stream(stream)))
    return cache


# --------------------------------------------------------------------------- timing
class AttentionParamsC(C.Structure):
    _fields_ = [("dim", C.c_int32), ("eps", C.c_float), ("gamma", C.c_void_p), ("beta", C.c_void_p),
                ("w_qkv", C.c_void_p), ("b_qkv", C.c_void_p), ("w_o", C.c_void_p),
                ("b_o", C.c_void_p)]


class AttentionBlock:
    """Device-resident parameters of the decoder mid-block attention block
    (``wanvae_attention_block``): bf16 projection weights, fp32 norm and biases."""

    def __init__(self, dim, gamma, beta, w_qkv, b_qkv, w_o, b_o, eps: float = EPS):
        self.dim, self.eps = int(dim), float(eps)
        self.tensors = dict(gamma=gamma, beta=beta, w_qkv=w_qkv, b_qkv=b_qkv, w_o=w_o, b_o=b_o)
        t = self.tensors
        self.c = AttentionParamsC(self.dim, self.eps, _ptr(t["gamma"]), _ptr(t["beta"]),
                                  _ptr(t["w_qkv"]), _ptr(t["b_qkv"]), _ptr(t["w_o"]), _ptr(t["b_o"]))

    @classmethod
    def from_host(cls, p: dict, device="cuda", eps: float = EPS):
        """From float32 numpy arrays gamma, beta, wqkv [3C, C], bqkv, wo [C, C], bo."""
        torch = _torch()
        f32 = lambda a: None if a is None else torch.from_numpy(a).to(device)
        bf = lambda a: torch.from_numpy(a).to(device).to(torch.bfloat16).contiguous()
        C_ = int(p["gamma"].shape[0])
        return cls(C_, f32(p["gamma"]), f32(p.get("beta")), bf(p["wqkv"]), f32(p.get("bqkv")),
                   bf(p["wo"]), f32(p.get("bo")), eps)

    def workspace_size(self, n, t, h, w) -> int:
        d = Dims(n, t, h, w)
        b = C.c_size_t(0)
        _check(lib().wanvae_attention_workspace_size(C.byref(self.c), C.byref(d), C.byref(b)))
        return b.value

    def workspace(self, n, t, h, w, device="cuda"):
        torch = _torch()
        return torch.empty(max(self.workspace_size(n, t, h, w), 1), dtype=torch.uint8, device=device)

    def forward(self, x, out=None, workspace=None, stream=None):
        """x [n,t,h,w,dim] bf16 -> y, the block's output."""
        torch = _torch()
        n, t, h, w, c = x.shape
        _dev(x, "x", torch.bfloat16, (n, t, h, w, self.dim))
        y = torch.empty_like(x) if out is None else out
        _dev(y, "out", torch.bfloat16, (n, t, h, w, self.dim))
        ws = self.workspace(n, t, h, w, x.device) if workspace is None else workspace
        d = Dims(n, t, h, w)
        _check(lib().wanvae_attention_block(C.byref(self.c), _ptr(x), _ptr(y), C.byref(d), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)))
        return y


def stream_copy(src, dst, unroll: int = 4, blocks_per_cu: int = 8, stream=None):
    """dst = src by the library's plain streaming copy (``wanvae_stream_copy``),
    the attainable HBM rate of its bandwidth-bound kernels.  Both GPU tensors,
    contiguous, of equal byte size (a multiple of 16)."""
    _dev(src, "src")
    _dev(dst, "dst")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must have the same byte size")
    _check(lib().wanvae_stream_copy(_ptr(src), _ptr(dst), nb, int(unroll), int(blocks_per_cu), _stream(stream)))
    return dst


def wait_giveups() -> int:
    """Bounded flag waits of the conv kernels that gave up on the current
    device since load or the last reset (``wanvae_wait_giveups``; waits for
    the device to go idle).  Zero when every launch kept its protocol."""
    n = C.c_uint64(0)
    _check(lib().wanvae_wait_giveups(C.byref(n)))
    return n.value


def wait_giveups_reset():
    _check(lib().wanvae_wait_giveups_reset())


def set_wait_bound(polls: int):
    """Polls before a flag wait gives up, for later launches; negative
    restores the default (``wanvae_set_wait_bound``; a test hook)."""
    _check(lib().wanvae_set_wait_bound(int(polls)))


def timing_enable(on: bool = True):
    _check(lib().wanvae_timing_enable(1 if on else 0))


def timing_reset():
    _check(lib().wanvae_timing_reset())


def timing_read(kind: int):
    """(launches, total_ms) of one kernel kind since the last reset."""
    n = C.c_int64(0)
    ms = C.c_double(0.0)
    _check(lib().wanvae_timing_read(kind, C.byref(n), C.byref(ms)))
    return n.value, ms.value
