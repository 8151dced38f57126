"""The conv kernel's tile decode, on the CPU.  It divides 31-bit work-item
indices by launch constants with a multiply and a shift (s = ceil(log2 d),
m = ceil(2^(31+s)/d), q = (n m) >> (31 + s)): the claim that this is exact for
0 <= n < 2^31 and 1 <= d < 2^31, and that m fits 32 bits, is checked over every
divisor up to 4096 and the edges above.  And its frame super-block order must
visit every (frame group, column block) of a row block exactly once, with a
ragged last super-block too."""
import numpy as np


def magic(d):
    s = 0
    while (1 << s) < d:
        s += 1
    return ((1 << (31 + s)) + d - 1) // d, s


def check(d, ns):
    m, s = magic(d)
    assert 0 < m < (1 << 32), (d, m)
    for n in ns:
        assert (n * m) >> (31 + s) == n // d, (n, d)


def test_every_small_divisor():
    top = (1 << 31) - 1
    for d in range(1, 4097):
        # around each multiple of d near 0 and near the top of the range, and
        # the largest index
        k = top // d
        ns = {0, 1, d - 1, d, d + 1, 2 * d - 1, top, k * d, k * d - 1, (k - 1) * d + d - 1}
        check(d, [n for n in ns if 0 <= n <= top])


def test_large_divisors_random_indices():
    rng = np.random.default_rng(0)
    top = (1 << 31) - 1
    ds = [4097, 65535, 65536, 65537, 194400, (1 << 30) - 1, 1 << 30, (1 << 30) + 1, top]
    ds += [int(v) for v in rng.integers(1, top, 200)]
    for d in ds:
        ns = [int(v) for v in rng.integers(0, top, 200)] + [top, d - 1, d, top - top % d, top - top % d - 1]
        check(d, [n for n in ns if 0 <= n <= top])


def decode_region(idx, ngroups, tiles_w, sbg):
    """The conv kernel's order within one (batch item, row block): frame groups
    in super-blocks of sbg (the last one shorter), the frame group fastest
    inside a super-block, then the column block.  Returns (group, column)."""
    nsb = (ngroups + sbg - 1) // sbg
    gw, full, last0 = sbg * tiles_w, (nsb - 1) * sbg * tiles_w, (nsb - 1) * sbg
    r = ngroups - last0
    if idx < full:
        s, rem = divmod(idx, gw)
        w, g = divmod(rem, sbg)
        return s * sbg + g, w
    w, g = divmod(idx - full, r)
    return last0 + g, w


def test_super_block_order_visits_every_tile_once():
    for ngroups in (1, 2, 19, 20, 21, 26, 80):
        for tiles_w in (1, 3, 40):
            for sbg in sorted({1, 7, 20, ngroups}):
                if sbg > ngroups:
                    continue
                seen = [decode_region(i, ngroups, tiles_w, sbg) for i in range(ngroups * tiles_w)]
                assert sorted(seen) == [(g, w) for g in range(ngroups) for w in range(tiles_w)]
    # one super-block is the plain order: frame group fastest, then column
    assert [decode_region(i, 5, 3, 5) for i in range(15)] == [(g, w) for w in range(3) for g in range(5)]
