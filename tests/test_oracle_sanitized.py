"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; gcc): every entry point runs on small inputs in a child
process with the sanitized build, which must finish clean and return the same
bits as the normal build (the sanitizers change no arithmetic: -ffp-contract=off
and fp64 sums in source order either way)."""
import os
import shutil
import subprocess
import sys
import textwrap

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    out = {{}}
    r = np.random.default_rng(11)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    x = f(1, 4, 5, 7, 16)
    g, b = (1 + 0.1 * f(16)), 0.1 * f(16)
    out["norm"] = oracle.norm_silu(x, g, b)
    out["rms"] = oracle.rms_norm(x, g, b)
    w = f(8, 16, 3, 3, 3) * 0.1
    out["conv"] = oracle.causal_conv3d(x, w, 0.1 * f(8))
    out["conv_cache"] = oracle.causal_conv3d(x, w, 0.1 * f(8), f(1, 2, 5, 7, 16))
    out["pointwise"] = oracle.pointwise_conv(x, f(5, 16), f(5))
    blk = oracle.Block(1 + 0.1 * f(16), 0.1 * f(16), 0.1 * f(24, 16, 3, 3, 3), 0.1 * f(24),
                       1 + 0.1 * f(24), 0.1 * f(24), 0.1 * f(24, 24, 3, 3, 3), 0.1 * f(24),
                       0.2 * f(24, 16), 0.1 * f(24))
    out["block"] = oracle.resblock_full(blk, x)
    out["stream"] = oracle.resblock_stream(blk, x, t_step=1)
    out["shortcut"] = oracle.shortcut(blk, x)
    out["up2"] = oracle.upsample2d_conv(x, 0.1 * f(8, 16, 3, 3), 0.1 * f(8))
    out["up3"] = oracle.upsample3d_conv(x, 0.1 * f(8, 16, 3, 3), 0.1 * f(8))
    xa = f(1, 2, 3, 4, 16)
    out["attn"] = oracle.attention_block(xa, 1 + 0.1 * f(16), 0.1 * f(16), 0.2 * f(48, 16),
                                         0.1 * f(48), 0.2 * f(16, 16), 0.1 * f(16))
    np.savez({path!r}, **out)
    print("child done")
""")


def _run_child(path, env):
    code = CHILD.format(root=ROOT, path=path)
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no libasan for gcc")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    base = dict(os.environ, OMP_NUM_THREADS="2")
    base.pop("WANVAE_ORACLE_LIB", None)
    # the normal build, for the reference bits
    ref = _run_child(str(tmp_path / "ref.npz"), base)
    assert ref.returncode == 0, ref.stderr[-3000:]
    san_env = dict(base, WANVAE_ORACLE_LIB=lib, LD_PRELOAD=asan,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    san = _run_child(str(tmp_path / "san.npz"), san_env)
    assert san.returncode == 0 and "child done" in san.stdout, san.stderr[-3000:]
    assert "runtime error" not in san.stderr and "AddressSanitizer" not in san.stderr, san.stderr[-3000:]
    a, b = np.load(tmp_path / "ref.npz"), np.load(tmp_path / "san.npz")
    assert sorted(a.files) == sorted(b.files)
    for k in a.files:
        assert np.array_equal(a[k], b[k]), k
