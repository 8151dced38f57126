"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against one of: an independent brute-force loop,
a PyTorch CPU library routine in float64, a closed form, or an invariant the
pages rely on ("Sharding of WAN 2.2 VAE": output channels are independent,
C_in partial sums add up to the full conv, the channel sum of squares adds up
across channel shards, a halo of (k-1)/2 reproduces the whole conv; "Closing
the gap", section 1: full-T computes what the per-frame feat_cache loop
computes).
"""
import math

import numpy as np
import pytest

from tests import refs
from tests.refs import rel_err

RNG = np.random.default_rng(1234)


def rnd(*shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float32)


def block_params(cin, cout, shortcut=None, seed=7):
    r = np.random.default_rng(seed)
    f = np.float32
    p = dict(
        gamma1=r.uniform(0.5, 1.5, cin).astype(f), beta1=(r.standard_normal(cin) * 0.3).astype(f),
        wa=(r.standard_normal((cout, cin, 3, 3, 3)) / math.sqrt(27 * cin)).astype(f),
        ba=(r.standard_normal(cout) * 0.1).astype(f),
        gamma2=r.uniform(0.5, 1.5, cout).astype(f), beta2=(r.standard_normal(cout) * 0.3).astype(f),
        wb=(r.standard_normal((cout, cout, 3, 3, 3)) / math.sqrt(27 * cout)).astype(f),
        bb=(r.standard_normal(cout) * 0.1).astype(f), ws=None, bs=None)
    if shortcut or cin != cout:
        p["ws"] = (r.standard_normal((cout, cin)) / math.sqrt(cin)).astype(f)
        p["bs"] = (r.standard_normal(cout) * 0.1).astype(f)
    return p


def mk_block(orc, p):
    return orc.Block(p["gamma1"], p["beta1"], p["wa"], p["ba"], p["gamma2"], p["beta2"],
                     p["wb"], p["bb"], p["ws"], p["bs"])


# --------------------------------------------------------------------------- SiLU
def test_silu_special_values(orc):
    assert orc.silu(0.0) == 0.0
    for u in (-30.0, -3.5, -1.0, -1e-3, 1e-3, 0.5, 1.0, 2.0, 7.25, 40.0):
        # silu(u) - silu(-u) = u (sigmoid(u) + sigmoid(-u) = 1)
        assert abs((orc.silu(u) - orc.silu(-u)) - u) <= 1e-15 * max(1.0, abs(u))
    assert abs(orc.silu(50.0) - 50.0) < 1e-12 and abs(orc.silu(-50.0)) < 1e-18


def test_silu_matches_torch(orc):
    us = np.linspace(-12, 12, 97)
    ref = refs.torch_silu(us)
    got = np.array([orc.silu(u) for u in us])
    assert np.max(np.abs(got - ref)) <= 1e-15 * np.max(np.abs(ref))


# --------------------------------------------------------------------------- RMS_norm
@pytest.mark.parametrize("C", [1, 3, 64, 96, 384])
def test_norm_unit_rms(orc, C):
    x = rnd(50, C, scale=3.0)
    u = orc.rms_norm(x, np.ones(C, np.float32), None).astype(np.float64)
    # gamma = 1, beta = 0: every channel vector has mean square 1
    assert np.all(np.abs((u * u).sum(-1) - C) <= 1e-5 * C)


def test_norm_affine_closed_form(orc):
    C = 96
    x = rnd(40, C)
    g = RNG.uniform(0.5, 1.5, C).astype(np.float32)
    b = rnd(C, scale=0.3)
    u = orc.rms_norm(x, g, b).astype(np.float64)
    z = (u - b) / g                   # undo the affine part: unit RMS again
    assert np.all(np.abs((z * z).mean(-1) - 1.0) <= 1e-5)
    # and the direction is x's own direction
    cos = (z * x).sum(-1) / np.linalg.norm(z, axis=-1) / np.linalg.norm(x.astype(np.float64), axis=-1)
    assert np.all(cos > 1 - 1e-6)


def test_norm_matches_torch_normalize(orc):
    C = 192
    x = rnd(64, C, scale=2.0)
    g = RNG.uniform(0.5, 1.5, C).astype(np.float32)
    b = rnd(C, scale=0.3)
    ref = refs.torch_norm(x, g, b)
    assert rel_err(orc.rms_norm(x, g, b), ref) <= 2e-7
    ref_s = refs.torch_silu(ref)
    assert rel_err(orc.norm_silu(x, g, b), ref_s) <= 2e-7


def test_norm_scale_invariance_bitwise(orc):
    C = 96
    x = rnd(30, C)
    g = RNG.uniform(0.5, 1.5, C).astype(np.float32)
    b = rnd(C)
    for k in (-8, -1, 3, 20):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        assert np.array_equal(orc.rms_norm(xs, g, b), orc.rms_norm(x, g, b))
        assert np.array_equal(orc.norm_silu(xs, g, b), orc.norm_silu(x, g, b))


def test_norm_zero_vector_gives_beta(orc):
    C = 64
    g = RNG.uniform(0.5, 1.5, C).astype(np.float32)
    b = rnd(C)
    z = np.zeros((3, C), np.float32)
    assert np.array_equal(orc.rms_norm(z, g, b), np.broadcast_to(b, (3, C)))
    expect = np.array([orc.silu(float(v)) for v in b], np.float64).astype(np.float32)
    assert np.array_equal(orc.norm_silu(z, g, b), np.broadcast_to(expect, (3, C)))


def test_norm_single_channel_is_sign(orc):
    # C = 1: x / |x| = +-1 exactly, so u = +-gamma + beta
    x = np.array([[3.0], [-0.25], [1e-10], [-7e5]], np.float32)
    g = np.array([1.25], np.float32)
    b = np.array([-0.5], np.float32)
    u = orc.rms_norm(x, g, b)
    expect = (np.sign(x.astype(np.float64)) * 1.25 - 0.5).astype(np.float32)
    assert np.array_equal(u, expect)
    # below eps the clamp takes over: u = x / eps * gamma + beta
    tiny = np.array([[1e-20]], np.float32)
    expect_tiny = np.float32(float(tiny[0, 0]) / 1e-12 * 1.25 - 0.5)
    assert orc.rms_norm(tiny, g, b)[0, 0] == expect_tiny


def test_norm_channel_shard_sums(orc):
    # the sum of squares runs over the whole channel axis: it is the sum of the
    # per-shard sums, so normalising one shard alone gives a different scale
    C = 384
    x = rnd(20, C)
    ones = np.ones(C, np.float32)
    u = orc.rms_norm(x, ones, None).astype(np.float64)
    xd = x.astype(np.float64)
    ss = sum((xd[:, s:s + 96] ** 2).sum(-1) for s in range(0, C, 96))
    expect = xd / np.sqrt(ss)[:, None] * math.sqrt(C)
    assert rel_err(u, expect) <= 2e-7
    half = orc.rms_norm(x[:, :192], ones[:192], None).astype(np.float64)
    assert rel_err(half, u[:, :192]) > 1e-3


# --------------------------------------------------------------------------- conv
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 1), (1, 2, 2, 5, 2, 3), (2, 4, 5, 2, 4, 2),
                                   (1, 4, 5, 5, 1, 1), (1, 1, 3, 3, 2, 2)])
def test_conv_bruteforce(orc, shape):
    N, T, H, W, Cin, Cout = shape
    x = rnd(N, T, H, W, Cin)
    w = rnd(Cout, Cin, 3, 3, 3)
    b = rnd(Cout)
    ref = refs.brute_conv(x, w, b)
    got = orc.causal_conv3d(x, w, b)
    assert rel_err(got, ref) <= 1e-7


def test_conv_bruteforce_with_cache(orc):
    N, T, H, W, Cin, Cout = 2, 2, 3, 4, 3, 2
    x = rnd(N, T, H, W, Cin)
    cache = rnd(N, 2, H, W, Cin)
    w = rnd(Cout, Cin, 3, 3, 3)
    b = rnd(Cout)
    assert rel_err(orc.causal_conv3d(x, w, b, cache), refs.brute_conv(x, w, b, cache)) <= 1e-7


@pytest.mark.parametrize("shape", [(1, 5, 7, 9, 8, 6), (2, 3, 4, 11, 16, 5), (1, 1, 6, 6, 4, 4)])
def test_conv_matches_torch_conv3d(orc, shape):
    N, T, H, W, Cin, Cout = shape
    x = rnd(N, T, H, W, Cin)
    w = rnd(Cout, Cin, 3, 3, 3, scale=0.2)
    b = rnd(Cout)
    assert rel_err(orc.causal_conv3d(x, w, b), refs.torch_conv(x, w, b)) <= 2e-7
    cache = rnd(N, 2, H, W, Cin)
    assert rel_err(orc.causal_conv3d(x, w, b, cache), refs.torch_conv(x, w, b, cache)) <= 2e-7


def test_conv_impulse_response(orc):
    # an impulse at (t0,h0,w0,ci0) reads back the kernel, exactly:
    # y[t,h,w,co] - b[co] = W[co, ci0, t0-t+2, h0-h+1, w0-w+1] inside the taps, else 0
    N, T, H, W, Cin, Cout = 1, 5, 6, 7, 3, 4
    w = rnd(Cout, Cin, 3, 3, 3)
    b = np.zeros(Cout, np.float32)
    for (t0, h0, w0, ci0) in [(0, 0, 0, 0), (2, 3, 4, 1), (4, 5, 6, 2), (1, 0, 6, 0)]:
        x = np.zeros((N, T, H, W, Cin), np.float32)
        x[0, t0, h0, w0, ci0] = 1.0
        y = orc.causal_conv3d(x, w, b)
        expect = np.zeros_like(y)
        for t in range(T):
            for h in range(H):
                for ww in range(W):
                    kt, kh, kw = t0 - t + 2, h0 - h + 1, w0 - ww + 1
                    if 0 <= kt < 3 and 0 <= kh < 3 and 0 <= kw < 3:
                        expect[0, t, h, ww] = w[:, ci0, kt, kh, kw]
        assert np.array_equal(y, expect)


def test_conv_constant_input(orc):
    N, T, H, W, Cin, Cout = 1, 4, 5, 6, 8, 3
    c = 0.5
    x = np.full((N, T, H, W, Cin), c, np.float32)
    w = rnd(Cout, Cin, 3, 3, 3)
    b = rnd(Cout)
    y = orc.causal_conv3d(x, w, b).astype(np.float64)
    wd = w.astype(np.float64)
    interior = b + c * wd.sum(axis=(1, 2, 3, 4))
    first = b + c * wd[:, :, 2].sum(axis=(1, 2, 3))     # frame 0: only kt = 2 sees data
    second = b + c * wd[:, :, 1:].sum(axis=(1, 2, 3, 4))
    tol = 1e-6 * np.abs(wd).sum()
    assert np.all(np.abs(y[0, 2:, 1:-1, 1:-1] - interior) <= tol)
    assert np.all(np.abs(y[0, 0, 1:-1, 1:-1] - first) <= tol)
    assert np.all(np.abs(y[0, 1, 1:-1, 1:-1] - second) <= tol)
    corner = b + c * wd[:, :, :, 1:, 1:].sum(axis=(1, 2, 3, 4))   # (t>=2, h=0, w=0)
    assert np.all(np.abs(y[0, 3, 0, 0] - corner) <= tol)


def test_conv_linearity(orc):
    x1, x2 = rnd(1, 3, 5, 6, 4), rnd(1, 3, 5, 6, 4)
    w = rnd(3, 4, 3, 3, 3)
    lhs = orc.causal_conv3d((2.0 * x1 - 0.5 * x2).astype(np.float32), w).astype(np.float64)
    rhs = 2.0 * orc.causal_conv3d(x1, w).astype(np.float64) - 0.5 * orc.causal_conv3d(x2, w)
    assert rel_err(lhs, rhs) <= 1e-6


def test_conv_output_channel_independence(orc):
    # column-parallel split: each output channel depends on its own filter only
    x = rnd(1, 3, 4, 5, 6)
    w = rnd(8, 6, 3, 3, 3)
    b = rnd(8)
    full = orc.causal_conv3d(x, w, b)
    for s in (slice(0, 3), slice(3, 8), slice(5, 6)):
        assert np.array_equal(orc.causal_conv3d(x, w[s], b[s]), full[..., s])


def test_conv_input_channel_partial_sums(orc):
    # row-parallel split: partial convs over C_in shards add up to the whole conv
    x = rnd(1, 3, 4, 5, 8)
    w = rnd(5, 8, 3, 3, 3)
    full = orc.causal_conv3d(x, w).astype(np.float64)
    parts = sum(orc.causal_conv3d(x[..., s:s + 2], w[:, s:s + 2]).astype(np.float64)
                for s in range(0, 8, 2))
    assert rel_err(parts, full) <= 1e-6


def test_conv_zero_cache_equals_no_cache(orc):
    x = rnd(2, 3, 4, 4, 3)
    w = rnd(2, 3, 3, 3, 3)
    b = rnd(2)
    z = np.zeros((2, 2, 4, 4, 3), np.float32)
    assert np.array_equal(orc.causal_conv3d(x, w, b, z), orc.causal_conv3d(x, w, b))


def test_conv_cache_is_prepended_frames(orc):
    # with a cache, the conv equals the no-cache conv of [cache, x] minus the
    # first two output frames
    x = rnd(1, 3, 4, 5, 3)
    cache = rnd(1, 2, 4, 5, 3)
    w = rnd(2, 3, 3, 3, 3)
    b = rnd(2)
    whole = orc.causal_conv3d(np.concatenate([cache, x], axis=1), w, b)
    assert np.array_equal(orc.causal_conv3d(x, w, b, cache), whole[:, 2:])


# --------------------------------------------------------------------------- shortcut
def test_pointwise_conv_is_a_channel_matmul(orc):
    """post_quant_conv (1x1x1): against an fp64 matmul, with and without bias,
    for a batch of positions of any leading shape."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 3, 4, 16)).astype(np.float32)
    w = rng.standard_normal((5, 16)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    want = np.einsum("...i,oi->...o", x.astype(np.float64), w.astype(np.float64)) + b
    got = orc.pointwise_conv(x, w, b)
    assert got.shape == (2, 3, 4, 5)
    assert np.array_equal(got, want.astype(np.float32))
    want0 = np.einsum("...i,oi->...o", x.astype(np.float64), w.astype(np.float64))
    assert np.array_equal(orc.pointwise_conv(x, w, None), want0.astype(np.float32))


def test_shortcut_identity_and_matmul(orc):
    p = block_params(6, 6)
    x = rnd(1, 2, 3, 4, 6)
    blk = mk_block(orc, p)
    assert np.array_equal(orc.shortcut(blk, x), x)
    p2 = block_params(6, 4)
    blk2 = mk_block(orc, p2)
    ref = x.astype(np.float64) @ p2["ws"].astype(np.float64).T + p2["bs"]
    assert rel_err(orc.shortcut(blk2, x), ref) <= 1e-7


# --------------------------------------------------------------------------- block
@pytest.mark.parametrize("cin,cout,shape", [(8, 8, (1, 4, 5, 6)), (8, 4, (2, 3, 4, 5)),
                                            (4, 12, (1, 2, 3, 3)), (16, 16, (1, 1, 2, 9))])
def test_block_matches_library_composition(orc, cin, cout, shape):
    p = block_params(cin, cout)
    x = rnd(*shape, cin)
    ref, _, _ = refs.torch_block(p, x)
    assert rel_err(orc.resblock_full(mk_block(orc, p), x), ref) <= 2e-6


def test_block_zero_convs_is_identity(orc):
    # WA = WB = 0 with zero biases and beta2 = 0: the residual branch is
    # silu(beta2) convolved with zero weights = 0, so y = x exactly
    p = block_params(8, 8)
    p.update(wa=np.zeros_like(p["wa"]), ba=np.zeros_like(p["ba"]), beta2=np.zeros_like(p["beta2"]),
             wb=np.zeros_like(p["wb"]), bb=np.zeros_like(p["bb"]))
    x = rnd(1, 3, 4, 5, 8)
    assert np.array_equal(orc.resblock_full(mk_block(orc, p), x), x)


def test_block_residual_reads_original_input(orc):
    # WB = 0, bB = c: y = round(x + c) whatever conv A does
    p = block_params(8, 8)
    c = 0.375
    p.update(wb=np.zeros_like(p["wb"]), bb=np.full(8, c, np.float32))
    x = rnd(1, 3, 4, 5, 8)
    expect = (x.astype(np.float64) + c).astype(np.float32)
    assert np.array_equal(orc.resblock_full(mk_block(orc, p), x), expect)
    # and with a 1x1 shortcut: y = round(Ws x + bs + c)
    p2 = block_params(8, 4)
    p2.update(wb=np.zeros_like(p2["wb"]), bb=np.full(4, c, np.float32))
    ref = x.astype(np.float64) @ p2["ws"].astype(np.float64).T + p2["bs"] + c
    assert rel_err(orc.resblock_full(mk_block(orc, p2), x), ref) <= 1e-7


# --------------------------------------------------------------------------- streaming
@pytest.mark.parametrize("cin,cout,shape,steps", [(8, 8, (1, 6, 5, 6), (1, 2, 3, 4, 6)),
                                                  (12, 4, (2, 5, 4, 3), (1, 2, 5))])
def test_stream_equals_full_bitwise(orc, cin, cout, shape, steps):
    p = block_params(cin, cout)
    blk = mk_block(orc, p)
    x = rnd(*shape, cin)
    full = orc.resblock_full(blk, x)
    for ts in steps:
        assert np.array_equal(orc.resblock_stream(blk, x, ts), full), f"t_step={ts}"


def test_stream_step_cache_contents(orc):
    # after each step the caches hold the last two frames of each conv's input
    p = block_params(8, 8)
    blk = mk_block(orc, p)
    x = rnd(1, 5, 3, 4, 8)
    _, n1, n2 = refs.torch_block(p, x)
    ca = np.zeros((1, 2, 3, 4, 8), np.float32)
    cb = np.zeros((1, 2, 3, 4, 8), np.float32)
    for t in range(5):
        orc.resblock_stream_step(blk, x[:, t:t + 1], ca, cb)
        for j, tt in enumerate((t - 1, t)):
            ea = n1[:, tt] if tt >= 0 else np.zeros_like(ca[:, 0])
            assert rel_err(ca[:, j], ea) <= 1e-6
        assert rel_err(cb[:, 1], n2[:, t]) <= 1e-5


def test_stream_resume_from_saved_caches(orc):
    # the caches are the only stream state: copying them out and resuming from
    # the copies continues bit for bit
    p = block_params(8, 4)
    blk = mk_block(orc, p)
    x = rnd(1, 6, 3, 5, 8)
    ca = np.zeros((1, 2, 3, 5, 8), np.float32)
    cb = np.zeros((1, 2, 3, 5, 4), np.float32)
    ys = [orc.resblock_stream_step(blk, x[:, t:t + 1], ca, cb) for t in range(3)]
    ca2, cb2 = ca.copy(), cb.copy()
    ys += [orc.resblock_stream_step(blk, x[:, t:t + 1], ca2, cb2) for t in range(3, 6)]
    assert np.array_equal(np.concatenate(ys, axis=1), orc.resblock_full(blk, x))


# --------------------------------------------------------------------------- window
@pytest.mark.parametrize("box", [(0, 2, 0, 2, 0, 3), (3, 7, 2, 5, 1, 4), (5, 7, 4, 6, 6, 9),
                                 (0, 7, 0, 6, 0, 9), (6, 7, 0, 1, 8, 9)])
def test_window_equals_full_bitwise(orc, box):
    p = block_params(8, 4)
    blk = mk_block(orc, p)
    T, H, W = 7, 6, 9
    x = rnd(2, T, H, W, 8)
    full = orc.resblock_full(blk, x)
    reg = orc.receptive_region(box, (T, H, W))
    xr = x[:, reg[0]:reg[1], reg[2]:reg[3], reg[4]:reg[5]]
    got = orc.resblock_window(blk, xr, reg, (T, H, W), box)
    t0, t1, h0, h1, w0, w1 = box
    assert np.array_equal(got, full[:, t0:t1, h0:h1, w0:w1])


# --------------------------------------------------------------------------- attention
def _attn_params(rng, C, scale=1.0):
    g = rng.uniform(0.5, 1.5, C).astype(np.float32)
    b = (rng.standard_normal(C) * 0.3).astype(np.float32)
    wqkv = (rng.standard_normal((3 * C, C)) * scale / np.sqrt(C)).astype(np.float32)
    bqkv = (rng.standard_normal(3 * C) * 0.1).astype(np.float32)
    wo = (rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32)
    bo = (rng.standard_normal(C) * 0.1).astype(np.float32)
    return g, b, wqkv, bqkv, wo, bo


def _attn_torch(x, g, b, wqkv, bqkv, wo, bo):
    """The same block from library routines in fp64: F.normalize for the norm,
    scaled_dot_product_attention (one head, default 1/sqrt(C) scale), matmul."""
    import torch
    N, T, H, W, C = x.shape
    X = torch.from_numpy(x).double()
    t = lambda a: torch.from_numpy(a).double()
    u = torch.nn.functional.normalize(X, dim=-1, eps=1e-12) * C ** 0.5 * t(g) + t(b)
    q, k, v = (u @ t(wqkv).T + t(bqkv)).split(C, -1)
    shp = (N * T, 1, H * W, C)
    o = torch.nn.functional.scaled_dot_product_attention(q.reshape(shp), k.reshape(shp), v.reshape(shp))
    return (X + (o.reshape(N, T, H, W, C) @ t(wo).T + t(bo))).numpy()


@pytest.mark.parametrize("shape", [(1, 2, 3, 5, 8), (2, 1, 4, 4, 16), (1, 3, 1, 7, 4)])
def test_attention_matches_library_routines(orc, shape):
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal(shape).astype(np.float32)
    p = _attn_params(rng, shape[-1], scale=2.0)
    y = orc.attention_block(x, *p)
    ref = _attn_torch(x, *p)
    assert np.abs(y - ref).max() <= 2e-6 * np.abs(ref).max()


def test_attention_zero_output_projection_is_identity(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 2, 3, 4, 8)).astype(np.float32)
    g, b, wqkv, bqkv, wo, bo = _attn_params(rng, 8)
    y = orc.attention_block(x, g, b, wqkv, bqkv, np.zeros_like(wo), np.zeros_like(bo))
    assert np.array_equal(y, x)


def test_attention_constant_values(orc):
    """v = c at every position (value weights 0, value bias c): any softmax
    weights average to c, so y = x + wo c + bo whatever q and k are."""
    rng = np.random.default_rng(2)
    C = 8
    x = rng.standard_normal((1, 2, 3, 4, C)).astype(np.float32)
    g, b, wqkv, bqkv, wo, bo = _attn_params(rng, C)
    wqkv[2 * C:] = 0.0
    c = rng.standard_normal(C).astype(np.float32)
    bqkv[2 * C:] = c
    y = orc.attention_block(x, g, b, wqkv, bqkv, wo, bo)
    want = x.astype(np.float64) + (wo.astype(np.float64) @ c.astype(np.float64) + bo)
    assert np.abs(y - want).max() <= 1e-6 * np.abs(want).max()


def test_attention_uniform_scores_average_values(orc):
    """k = 0 (key weights and bias 0): every score is 0, the softmax is uniform
    and o is the mean of v over the frame's positions."""
    rng = np.random.default_rng(3)
    C, H, W = 8, 3, 5
    x = rng.standard_normal((1, 2, H, W, C)).astype(np.float32)
    g, b, wqkv, bqkv, wo, bo = _attn_params(rng, C)
    wqkv[C:2 * C] = 0.0
    bqkv[C:2 * C] = 0.0
    y = orc.attention_block(x, g, b, wqkv, bqkv, wo, bo)
    u = orc.rms_norm(x, g, b).astype(np.float64)
    v = u @ wqkv[2 * C:].astype(np.float64).T + bqkv[2 * C:]
    mean_v = v.mean(axis=(2, 3), keepdims=True)
    want = x + mean_v @ wo.astype(np.float64).T + bo
    assert np.abs(y - want).max() <= 1e-5 * np.abs(want).max()


def test_attention_single_position_returns_its_value(orc):
    """One position per frame: the softmax has one term, o = v."""
    rng = np.random.default_rng(4)
    C = 16
    x = rng.standard_normal((1, 3, 1, 1, C)).astype(np.float32)
    g, b, wqkv, bqkv, wo, bo = _attn_params(rng, C)
    y = orc.attention_block(x, g, b, wqkv, bqkv, wo, bo)
    u = orc.rms_norm(x, g, b).astype(np.float64)
    v = u @ wqkv[2 * C:].astype(np.float64).T + bqkv[2 * C:]
    want = x + v @ wo.astype(np.float64).T + bo
    assert np.abs(y - want).max() <= 1e-5 * np.abs(want).max()


def test_attention_frames_are_independent(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 3, 4, 8)).astype(np.float32)
    p = _attn_params(rng, 8)
    y = orc.attention_block(x, *p)
    x2 = x.copy()
    x2[1, 2] += 1.0
    x2[0, 0] *= 3.0
    y2 = orc.attention_block(x2, *p)
    assert np.array_equal(y2[0, 1:], y[0, 1:]) and np.array_equal(y2[1, :2], y[1, :2])
    assert not np.array_equal(y2[1, 2], y[1, 2])


def test_attention_permutation_equivariant(orc):
    """Permuting the positions of a frame permutes its output."""
    rng = np.random.default_rng(6)
    H, W, C = 3, 5, 8
    x = rng.standard_normal((1, 1, H, W, C)).astype(np.float32)
    p = _attn_params(rng, C)
    y = orc.attention_block(x, *p).reshape(H * W, C)
    perm = rng.permutation(H * W)
    xp = x.reshape(H * W, C)[perm].reshape(1, 1, H, W, C)
    yp = orc.attention_block(xp, *p).reshape(H * W, C)
    assert np.abs(yp - y[perm]).max() <= 1e-6 * np.abs(y).max()


def test_attention_sampled_queries_equal_full(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 2, 4, 6, 8)).astype(np.float32)
    p = _attn_params(rng, 8)
    y = orc.attention_block(x, *p)
    q = [23, 0, 7, 7, 11]
    ys = orc.attention_block(x, *p, frame=(0, 1), queries=q)
    assert np.array_equal(ys, y[0, 1].reshape(-1, 8)[q])


# --------------------------------------------------------------------------- upsample2d
def _up_params(rng, cin, cout):
    w = (rng.standard_normal((cout, cin, 3, 3)) / np.sqrt(9 * cin)).astype(np.float32)
    b = (rng.standard_normal(cout) * 0.1).astype(np.float32)
    return w, b


@pytest.mark.parametrize("shape,cout", [((1, 2, 3, 5, 8), 4), ((2, 1, 4, 4, 16), 8), ((1, 1, 1, 1, 3), 5)])
def test_upsample2d_matches_library_routines(orc, shape, cout):
    """torch fp64: F.interpolate(scale_factor=2, mode='nearest') then
    F.conv2d(padding=1), frame by frame."""
    import torch
    rng = np.random.default_rng(sum(shape) + cout)
    x = rng.standard_normal(shape).astype(np.float32)
    w, b = _up_params(rng, shape[-1], cout)
    y = orc.upsample2d_conv(x, w, b)
    N, T, H, W, C = shape
    X = torch.from_numpy(x).double().reshape(N * T, H, W, C).permute(0, 3, 1, 2)
    U = torch.nn.functional.interpolate(X, scale_factor=2, mode="nearest")
    R = torch.nn.functional.conv2d(U, torch.from_numpy(w).double(), torch.from_numpy(b).double(), padding=1)
    ref = R.permute(0, 2, 3, 1).reshape(N, T, 2 * H, 2 * W, cout).numpy()
    assert y.shape == ref.shape
    assert np.abs(y - ref).max() <= 1e-6 * np.abs(ref).max()


def test_upsample2d_brute_force(orc):
    """Pure-Python loops over the definition, with explicit bounds checks."""
    rng = np.random.default_rng(5)
    H, W, cin, cout = 2, 3, 2, 3
    x = rng.standard_normal((1, 1, H, W, cin)).astype(np.float32)
    w, b = _up_params(rng, cin, cout)
    y = orc.upsample2d_conv(x, w, b)
    for h in range(2 * H):
        for c in range(2 * W):
            for co in range(cout):
                acc = float(b[co])
                for kh in range(3):
                    for kw in range(3):
                        uh, uw = h + kh - 1, c + kw - 1
                        if 0 <= uh < 2 * H and 0 <= uw < 2 * W:
                            for ci in range(cin):
                                acc += float(w[co, ci, kh, kw]) * float(x[0, 0, uh // 2, uw // 2, ci])
                assert abs(y[0, 0, h, c, co] - acc) <= 1e-6 * (1 + abs(acc))


def test_upsample2d_equals_conv3d_current_tap_on_repeated_input(orc):
    """Against the pinned causal conv: the frames repeated 2x2 (np.repeat)
    through a 3x3x3 conv whose only nonzero temporal tap is the current
    frame's give the same sums in the same order: bitwise equal."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 3, 4, 5, 16)).astype(np.float32)
    w, b = _up_params(rng, 16, 8)
    up = np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)
    w3 = np.zeros((8, 16, 3, 3, 3), np.float32)
    w3[:, :, 2] = w
    ref = orc.causal_conv3d(up, w3, b)
    y = orc.upsample2d_conv(x, w, b)
    assert np.array_equal(y, ref)


def test_upsample2d_centre_tap_gives_2x2_blocks(orc):
    """Only the centre tap: each input position becomes a 2x2 block of one
    value, the pointwise conv of that position."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 2, 3, 4, 16)).astype(np.float32)
    w, b = _up_params(rng, 16, 8)
    wc = np.zeros_like(w)
    wc[:, :, 1, 1] = w[:, :, 1, 1]
    y = orc.upsample2d_conv(x, wc, b)
    pw = orc.pointwise_conv(x, np.ascontiguousarray(w[:, :, 1, 1]), b)
    for a in range(2):
        for c in range(2):
            assert np.array_equal(y[:, :, a::2, c::2], pw)


def test_upsample2d_constant_input(orc):
    """x = c everywhere: the interior sees all 9 taps, the top-left corner the
    four taps kh, kw in {1, 2}, the right edge the six taps kw in {0, 1}."""
    rng = np.random.default_rng(8)
    cin, cout, c = 8, 4, 0.75
    x = np.full((1, 1, 3, 3, cin), c, np.float32)
    w, b = _up_params(rng, cin, cout)
    y = orc.upsample2d_conv(x, w, b).astype(np.float64)
    s = w.astype(np.float64).sum(axis=1)                       # [cout, 3, 3]
    np.testing.assert_allclose(y[0, 0, 2, 2], b + c * s.sum(axis=(1, 2)), rtol=1e-6)
    np.testing.assert_allclose(y[0, 0, 0, 0], b + c * s[:, 1:, 1:].sum(axis=(1, 2)), rtol=1e-6)
    np.testing.assert_allclose(y[0, 0, 3, 5], b + c * s[:, :, :2].sum(axis=(1, 2)), rtol=1e-6)


def test_upsample2d_rows_and_frames_equal_full(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 3, 5, 4, 16)).astype(np.float32)
    w, b = _up_params(rng, 16, 8)
    full = orc.upsample2d_conv(x, w, b)
    part = orc.upsample2d_conv(x, w, b, frames=[(1, 2), (0, 0)], rows=(3, 8))
    assert np.array_equal(part[0], full[1, 2, 3:8])
    assert np.array_equal(part[1], full[0, 0, 3:8])


# --------------------------------------------------------------------------- upsample3d
def _frames_doubled_after_first(x):
    """Frame 0 once, then every later frame twice, built with numpy's repeat:
    the frame sequence the temporal reading gives (T -> 2T - 1)."""
    return np.concatenate([x[:, :1], np.repeat(x[:, 1:], 2, axis=1)], axis=1)


@pytest.mark.parametrize("shape,cout", [((1, 3, 3, 5, 8), 4), ((2, 2, 4, 4, 16), 8), ((1, 1, 2, 3, 4), 3)])
def test_upsample3d_matches_library_routines(orc, shape, cout):
    """torch fp64: the frames doubled after the first (torch
    repeat_interleave), then F.interpolate(nearest, x2 in H and W) and
    F.conv2d(padding=1) per frame."""
    import torch
    rng = np.random.default_rng(sum(shape) + 3 * cout)
    x = rng.standard_normal(shape).astype(np.float32)
    w, b = _up_params(rng, shape[-1], cout)
    y = orc.upsample3d_conv(x, w, b)
    N, T, H, W, C = shape
    X = torch.from_numpy(x).double()
    X = torch.cat([X[:, :1], torch.repeat_interleave(X[:, 1:], 2, dim=1)], dim=1)   # [N, 2T-1, H, W, C]
    To = 2 * T - 1
    U = torch.nn.functional.interpolate(X.reshape(N * To, H, W, C).permute(0, 3, 1, 2), scale_factor=2,
                                        mode="nearest")
    R = torch.nn.functional.conv2d(U, torch.from_numpy(w).double(), torch.from_numpy(b).double(), padding=1)
    ref = R.permute(0, 2, 3, 1).reshape(N, To, 2 * H, 2 * W, cout).numpy()
    assert y.shape == ref.shape == (N, To, 2 * H, 2 * W, cout)
    assert np.abs(y - ref).max() <= 1e-6 * np.abs(ref).max()


def test_upsample3d_brute_force(orc):
    """Pure-Python loops: for output frame t', the input frame is looked up in
    an explicit list [0, 1, 1, 2, 2, ...]; bounds checked per tap."""
    rng = np.random.default_rng(12)
    T, H, W, cin, cout = 3, 2, 2, 2, 3
    x = rng.standard_normal((1, T, H, W, cin)).astype(np.float32)
    w, b = _up_params(rng, cin, cout)
    y = orc.upsample3d_conv(x, w, b)
    src = [0]
    for k in range(1, T):
        src += [k, k]
    assert y.shape[1] == len(src) == 5
    for tt, s in enumerate(src):
        for h in range(2 * H):
            for c in range(2 * W):
                for co in range(cout):
                    acc = float(b[co])
                    for kh in range(3):
                        for kw in range(3):
                            uh, uw = h + kh - 1, c + kw - 1
                            if 0 <= uh < 2 * H and 0 <= uw < 2 * W:
                                for ci in range(cin):
                                    acc += float(w[co, ci, kh, kw]) * float(x[0, s, uh // 2, uw // 2, ci])
                    assert abs(y[0, tt, h, c, co] - acc) <= 1e-6 * (1 + abs(acc))


def test_upsample3d_equals_upsample2d_of_doubled_frames(orc):
    """Bitwise equal to the pinned spatial upsampler on the frame sequence
    built by numpy's repeat; one frame in gives that frame's upsample2d."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 4, 3, 5, 16)).astype(np.float32)
    w, b = _up_params(rng, 16, 8)
    assert np.array_equal(orc.upsample3d_conv(x, w, b), orc.upsample2d_conv(_frames_doubled_after_first(x), w, b))
    assert np.array_equal(orc.upsample3d_conv(x[:, :1], w, b), orc.upsample2d_conv(x[:, :1], w, b))


def test_upsample3d_is_causal(orc):
    """A clip's first k + 1 frames give the first 2k + 1 output frames
    (bitwise), and changing input frame k changes output frames 2k - 1 and
    2k only (frame 0 for k = 0)."""
    rng = np.random.default_rng(14)
    T = 5
    x = rng.standard_normal((1, T, 3, 4, 16)).astype(np.float32)
    w, b = _up_params(rng, 16, 8)
    full = orc.upsample3d_conv(x, w, b)
    for k in range(T):
        assert np.array_equal(orc.upsample3d_conv(x[:, :k + 1], w, b), full[:, :2 * k + 1])
        xk = x.copy()
        xk[:, k] += 1.0
        yk = orc.upsample3d_conv(xk, w, b)
        changed = [t for t in range(2 * T - 1) if not np.array_equal(yk[:, t], full[:, t])]
        assert changed == ([0] if k == 0 else [2 * k - 1, 2 * k])
