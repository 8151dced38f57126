"""The oracle still reproduces its frozen output on the fp32 workload."""
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_frozen_c1_samples():
    y = make_golden.compute()
    rows = [l.split() for l in open(make_golden.OUT) if not l.startswith("#")]
    assert len(rows) == len(make_golden.SAMPLES)
    for t, h, w, c, bits, _ in rows:
        got = np.float32(y[0, int(t), int(h), int(w), int(c)]).view(np.uint32)
        assert got == int(bits, 16), (t, h, w, c)
