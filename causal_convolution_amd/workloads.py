"""Seeded synthetic inputs for the ResidualBlock workloads.

This module holds the workload table and the random draws only; it contains
none of the block's arithmetic, so both the HIP path's harness and the CPU
oracle's tests may take inputs from it.

Shapes follow the Wan 2.2 decoder stages the pages describe ("Sharding of WAN
2.2 VAE", the decoder module tree: 384 channels at latent resolution, 192 and
96 after upsampling; "Closing the gap", gap #1: ~21 latent frames).  The pages
use trained weights and real video latents; none are available, so i.i.d.
draws of the same shapes stand in.  Distributions N(mu, v) are read with v the
variance (weights with variance 1/fan_in keep activations of order one).

Draw order is fixed: gamma1, beta1, conv A weight, conv A bias, gamma2, beta2,
conv B weight, conv B bias, shortcut weight, shortcut bias, all from
``numpy.random.default_rng(seed)``.  Conv weights are drawn in the pages'
order [C_out, C_in, kD, kH, kW]; in bf16 workloads they are rounded to bf16
(round to nearest even) so that the HIP path and the oracle see the same
values.  Norm scales/shifts and biases stay float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": activations and conv weights
    n: int
    t: int
    h: int
    w: int
    cin: int
    cout: int
    desc: str

    @property
    def dims(self):
        return (self.n, self.t, self.h, self.w)

    @property
    def positions(self):
        return self.n * self.t * self.h * self.w

    @property
    def identity_shortcut(self):
        return self.cin == self.cout


WORKLOADS = {
    "c1": Workload("c1", F32, 1, 4, 16, 16, 64, 64,
                   "single ResidualBlock, fp32, 64->64, [1,4,16,16,64], identity shortcut"),
    "c2": Workload("c2", BF16, 1, 21, 90, 160, 384, 384,
                   "latent-resolution ResidualBlock, bf16, 384->384, [1,21,90,160,384], full-T"),
    "c3": Workload("c3", BF16, 1, 41, 360, 640, 192, 192,
                   "mid-resolution ResidualBlock, bf16, 192->192, [1,41,360,640,192], full-T"),
    "c4": Workload("c4", BF16, 1, 81, 720, 1280, 96, 96,
                   "output-resolution ResidualBlock, bf16, 96->96, [1,81,720,1280,96], full-T"),
    "c5": Workload("c5", BF16, 1, 41, 180, 320, 384, 192,
                   "channel-changing ResidualBlock, bf16, 384->192 with 1x1x1 shortcut, "
                   "[1,41,180,320,384], full-T and streaming"),
}


def custom(name, dtype, n, t, h, w, cin, cout):
    """A workload of another shape with the same value recipe (tests, edge cases)."""
    return Workload(name, dtype, n, t, h, w, cin, cout, f"{name} {dtype} [{n},{t},{h},{w}] {cin}->{cout}")


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Done with torch's own float32->bfloat16 cast, which rounds to nearest even.
    """
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def make_params(wl: Workload, seed: int = 0):
    """Block parameters as float32 numpy arrays, conv weights in the pages' order.

    Returns a dict with gamma1, beta1, wa [cout,cin,3,3,3], ba, gamma2, beta2,
    wb [cout,cout,3,3,3], bb, and ws [cout,cin] / bs (None for an identity
    shortcut).
    """
    rng = np.random.default_rng(seed)
    ci, co = wl.cin, wl.cout
    f32 = np.float32

    def normal(var, shape):
        return rng.normal(0.0, np.sqrt(var), size=shape).astype(f32)

    p = {}
    p["gamma1"] = rng.uniform(0.5, 1.5, size=ci).astype(f32)
    p["beta1"] = normal(0.1, ci)
    p["wa"] = normal(1.0 / (ci * 27), (co, ci, 3, 3, 3))
    p["ba"] = normal(0.01, co)
    p["gamma2"] = rng.uniform(0.5, 1.5, size=co).astype(f32)
    p["beta2"] = normal(0.1, co)
    p["wb"] = normal(1.0 / (co * 27), (co, co, 3, 3, 3))
    p["bb"] = normal(0.01, co)
    if ci != co:
        p["ws"] = normal(1.0 / ci, (co, ci))
        p["bs"] = normal(0.01, co)
    else:
        p["ws"] = None
        p["bs"] = None
    if wl.dtype == BF16:
        for k in ("wa", "wb", "ws"):
            if p[k] is not None:
                p[k] = round_bf16(p[k])
    return p


def make_attention_params(C: int, seed: int = 0):
    """Attention-block parameters as float32 numpy arrays, drawn like the
    ResidualBlock's: gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1), projection weights
    ~ N(0, 1/C) (variance 1 / fan_in), biases ~ N(0, 0.01); the weights rounded
    to bf16 values.  Keys gamma, beta, wqkv [3C, C] (q, k, v rows), bqkv [3C],
    wo [C, C], bo [C]."""
    rng = np.random.default_rng(seed + 77)
    f32 = np.float32

    def normal(var, shape):
        return rng.normal(0.0, np.sqrt(var), size=shape).astype(f32)

    return {"gamma": rng.uniform(0.5, 1.5, size=C).astype(f32), "beta": normal(0.1, C),
            "wqkv": round_bf16(normal(1.0 / C, (3 * C, C))), "bqkv": normal(0.01, 3 * C),
            "wo": round_bf16(normal(1.0 / C, (C, C))), "bo": normal(0.01, C)}


def make_upsample_params(cin: int, cout: int, seed: int = 0):
    """Upsampler conv parameters as float32 numpy arrays: w [cout, cin, 3, 3]
    ~ N(0, 1/(9 cin)) (variance 1 / fan_in) rounded to bf16 values, b ~ N(0,
    0.01)."""
    rng = np.random.default_rng(seed + 91)
    w = rng.normal(0.0, np.sqrt(1.0 / (9 * cin)), size=(cout, cin, 3, 3)).astype(np.float32)
    b = rng.normal(0.0, 0.1, size=cout).astype(np.float32)
    return round_bf16(w), b


def make_x_host(wl: Workload, seed: int = 0) -> np.ndarray:
    """x ~ N(0, 1) as float32 [N,T,H,W,Cin] on the host (small workloads);
    rounded to bf16 values for bf16 workloads."""
    rng = np.random.default_rng(seed + 1_000_003)
    x = rng.standard_normal(size=(wl.n, wl.t, wl.h, wl.w, wl.cin), dtype=np.float32)
    if wl.dtype == BF16:
        x = round_bf16(x)
    return x


def make_x_device(wl: Workload, seed: int = 0, device="cuda"):
    """x ~ N(0, 1) drawn on the device with torch's generator, frame by frame
    (bounded temporaries for the 14 GB output-resolution tensor), stored in the
    workload's dtype.  Tests copy x back to the host to feed the oracle."""
    import torch
    dt = torch.bfloat16 if wl.dtype == BF16 else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty((wl.n, wl.t, wl.h, wl.w, wl.cin), dtype=dt, device=device)
    for n in range(wl.n):
        for t in range(wl.t):
            x[n, t].copy_(torch.randn((wl.h, wl.w, wl.cin), dtype=torch.float32, device=device,
                                      generator=g))
    return x
