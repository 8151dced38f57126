"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a temporary copy of ``oracle/oracle.c`` (a
flipped time index, a transposed weight index, a dropped bias or residual, a
wrong cache frame, ...), builds it, and runs the pin suite against the broken
build: at least one pin must fail.  Mistakes are planted in the CPU oracle
only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "anti_causal_time": ("field_ptr(z, cache, n, t + kt - 2,", "field_ptr(z, cache, n, t - kt,"),
    "time_offset_off_by_one": ("field_ptr(z, cache, n, t + kt - 2,", "field_ptr(z, cache, n, t + kt - 1,"),
    "kh_kw_transposed": ("* 9 + kh * 3 + kw]", "* 9 + kw * 3 + kh]"),
    "h_pad_shift": ("t + kt - 2, h + kh - 1,", "t + kt - 2, h + kh,"),
    "ci_co_transposed": ("wt[(((int64_t)co * cin + ci) * 3 + kt)", "wt[(((int64_t)ci * cin + co) * 3 + kt)"),
    "dropped_bias": ("v += bias ? (double)bias[co] : 0.0;", "v += 0.0;"),
    "norm_missing_sqrtC": ("/ d * sqrt((double)C) *", "/ d *"),
    "norm_mean_not_sum": ("double r = sqrt(ss);", "double r = sqrt(ss / C);"),
    "norm_dropped_beta": ("+ (beta ? (double)beta[c] : 0.0);", "+ 0.0;"),
    "silu_wrong_sign": ("return u / (1.0 + exp(-u));", "return u / (1.0 + exp(u));"),
    "dropped_residual": ("if (!p->ws) return (double)xp[co];", "if (!p->ws) return 0.0;"),
    "shortcut_weight_transposed": ("p->ws[(int64_t)co * p->cin + ci]", "p->ws[(int64_t)ci * p->cout + co]"),
    "shortcut_dropped_bias": ("return acc + (p->bs ? (double)p->bs[co] : 0.0);", "return acc;"),
    "cache_frames_swapped": ("cache + ((((n * 2 + (t + 2))", "cache + ((((n * 2 + (-1 - t))"),
    "cache_roll_wrong_slot": ("memcpy(c + slab, z, sizeof(float) * (size_t)slab);",
                              "memcpy(c, z, sizeof(float) * (size_t)slab);"),
    "cache_holds_raw_input": ("roll_cache(cache_a, n1, N, Tc, H, W, p->cin);",
                              "roll_cache(cache_a, x, N, Tc, H, W, p->cin);"),
    "window_halo_too_small": ("int64_t ah0 = max64(bh0 - 1, 0), ah1 = min64(bh1 + 1, H);",
                              "int64_t ah0 = bh0, ah1 = bh1;"),
    "attention_missing_scale": ("s[j] = d * scale;", "s[j] = d;"),
    "attention_not_normalised": ("o[c] = (float)(acc[c] / z);", "o[c] = (float)acc[c];"),
    "attention_dropped_residual": ("(float)((double)xi[co] + t +", "(float)(t +"),
    "attention_k_v_swapped": ("const float *wk = wqkv + ((int64_t)C + c) * C;",
                              "const float *wk = wqkv + ((int64_t)2 * C + c) * C;"),
    "attention_query_from_raw_input": ("sq += (double)wq[t] * (double)ui[t];",
                                       "sq += (double)wq[t] * (double)x[i * (int64_t)C + t];"),
    "upsample_rounds_up": ("xf + ((uh / 2) * W + uw / 2) * (int64_t)cin;",
                           "xf + ((uh / 2) * W + (uw + 1) / 2 % W) * (int64_t)cin;"),
    "upsample_pad_shift": ("const int64_t uh = h + kh - 1;", "const int64_t uh = h + kh;"),
    "upsample_kh_kw_transposed": ("* cin + ci) * 3 + kh) * 3 + kw]", "* cin + ci) * 3 + kw) * 3 + kh]"),
    "upsample_dropped_bias": ("if (b) acc += (double)b[co];", "if (b) acc += 0.0;"),
    "upsample_row_stride": ("xf + ((uh / 2) * W + uw / 2)", "xf + ((uh / 2) * 2 * W / 2 + uw / 2 + uh % 2)"),
    "upsample3d_frames_anti_causal": ("const int64_t src = (t + 1) / 2;", "const int64_t src = t / 2;"),
    "upsample3d_resize_nearest": ("const int64_t src = (t + 1) / 2;", "const int64_t src = t * T / To;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    msrc = tmp_path / "oracle_mutant.c"
    msrc.write_text(src.replace(old, new))
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build_to(str(tmp_path / "liboracle_mutant.so"), str(msrc))
    env = dict(os.environ, WANVAE_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
