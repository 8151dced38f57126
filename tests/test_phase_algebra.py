"""The upsampler conv by output phase, checked on the CPU.

After a nearest x2 doubling, the 3x3 taps of output row 2i + py land on input
rows i + py - 1 and i + py only, so each output phase (py, px) is a 2x2 conv
of the half-resolution input with merged weights.  This test writes that form
out in numpy (fp64, no rounding) and compares it with the oracle's direct
definition (double the image, then the 9 taps): the two agree to rounding,
which pins the merge sets the GPU's weight packing uses.  (The GPU then rounds
each merged weight to bf16 once; its parity tests hold it to the bf16 bar.)
"""
import numpy as np

import oracle

# kernel taps (0..2 for dy = -1..+1) merged into tap t of phase p
MERGE = {(0, 0): [0], (0, 1): [1, 2], (1, 0): [0, 1], (1, 1): [2]}


def phase_form(x, w, b):
    """x [n,t,h,w,cin], w [cout,cin,3,3], b [cout] -> [n,t,2h,2w,cout], fp64."""
    n, t, h, wd, cin = x.shape
    cout = w.shape[0]
    xp = np.zeros((n, t, h + 2, wd + 2, cin))
    xp[:, :, 1:-1, 1:-1] = x
    y = np.zeros((n, t, 2 * h, 2 * wd, cout))
    for py in (0, 1):
        for px in (0, 1):
            acc = np.zeros((n, t, h, wd, cout)) + b
            for a in (0, 1):
                for bb in (0, 1):
                    wm = sum(w[:, :, ky, kx] for ky in MERGE[(py, a)] for kx in MERGE[(px, bb)])  # [cout, cin]
                    # input row i + py - 1 + a (padded index i + py + a)
                    xs = xp[:, :, py + a:py + a + h, px + bb:px + bb + wd]
                    acc += xs @ wm.T
            y[:, :, py::2, px::2] = acc
    return y


def test_phase_form_equals_direct_upsample_conv():
    rng = np.random.default_rng(3)
    for (n, t, h, wd, cin, cout) in [(1, 2, 5, 7, 16, 8), (2, 1, 1, 1, 4, 3), (1, 1, 6, 3, 8, 5)]:
        x = rng.standard_normal((n, t, h, wd, cin)).astype(np.float32)
        w = rng.standard_normal((cout, cin, 3, 3)).astype(np.float32)
        b = rng.standard_normal(cout).astype(np.float32)
        ref = oracle.upsample2d_conv(x, w, b)
        got = phase_form(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
        assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()


def test_phase_form_catches_a_wrong_merge():
    """A merge set off by one (phase 0's second row tap without dy = +1)
    breaks the equality: the check above is sensitive to the sets."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 1, 4, 4, 4)).astype(np.float32)
    w = rng.standard_normal((3, 4, 3, 3)).astype(np.float32)
    b = np.zeros(3, np.float32)
    ref = oracle.upsample2d_conv(x, w, b)
    saved = MERGE[(0, 1)]
    try:
        MERGE[(0, 1)] = [1]
        got = phase_form(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    finally:
        MERGE[(0, 1)] = saved
    assert np.abs(got - ref).max() > 1e-2 * np.abs(ref).max()
