"""Throughput of the full-T Wan 2.2 VAE-decoder ResidualBlock on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one ``wanvae_resblock_forward`` over the whole clip (norm1, conv A,
norm2, conv B with the residual add), with x, weights, workspace and y already
resident in HBM.  The default workload is the largest one, the
output-resolution block: bf16, 96 -> 96 channels, x = [1, 81, 720, 1280, 96]
(14.3 GB per activation), seeded synthetic values; c1, c2, c3 and c5 run with
``--workload``.  W untimed steps, then two timed passes of K steps each: the
first with nothing but the steps between its two events gives ``value`` and
``ms_per_step``; the second brackets every library launch with hipEvents on
the launch stream and gives the per-kernel durations.  The run prints one
JSON line:

* value: frames per second (T * K / elapsed) of the uninstrumented pass;
* roofline: the conv kernel's achieved TFLOP/s (algorithmic FLOPs per launch,
  2 * P * C_out * 27 * C_in plus 2 * P * C_out * C_in for a 1x1x1 shortcut
  computed in the conv, divided by its average launch time in the
  instrumented pass) against the 2.5 PFLOP/s dense bf16 MFMA peak;
* norm: the fused RMS_norm + SiLU kernel's achieved GB/s (2 * P * C * 2 bytes
  per launch) against the 8 TB/s HBM peak ("hbm_valid" is false where its
  tensors fit the 256 MB Infinity Cache, as at c2);
* traffic (in roofline and norm): HBM bytes per launch measured by rocprofv3
  FETCH_SIZE / WRITE_SIZE passes (scaled by what they read for a plain copy of
  known size), from profiles/traffic.json; null once any library source or
  build flag differs from the ones it was measured on;
* wait_giveups: bounded flag waits of the conv that gave up during the run
  (0 unless a launch left its synchronisation protocol);
* cpu_baseline: the CPU oracle timed on this host on a bounded sample (the
  whole block over the clip's first frame(s); causal, so those frames are
  exactly the clip's first output frames), scaled to frames per second.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ResidualBlock frames/sec + conv TFLOP/s (% bf16 MFMA peak), full-T, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def conv_flops(w, shortcut_in_conv=True):
    """Algorithmic FLOPs of conv A and conv B (+ the 1x1x1 shortcut when conv
    B computes it in its own K loop)."""
    P = w.positions
    fa = 2.0 * P * w.cout * 27 * w.cin
    fb = 2.0 * P * w.cout * 27 * w.cout
    if w.cin != w.cout and shortcut_in_conv:
        fb += 2.0 * P * w.cout * w.cin
    return fa, fb


def norm_bytes(w, esize):
    P = w.positions
    return 2.0 * P * w.cin * esize, 2.0 * P * w.cout * esize


# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, kept in
# profiles/traffic.json with the sha256 of every library source and of the
# build script (which holds the compiler flags) it was measured on: reported
# only while all of them are unchanged (else null).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def library_sources():
    """Every file the HIP library is built from, relative to the repo root."""
    rels = ["causal_convolution_amd/build.py"]
    for d in ("causal_convolution_amd/csrc", "include"):
        for f in sorted(os.listdir(os.path.join(ROOT, d))):
            rels.append(f"{d}/{f}")
    return rels


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in library_sources():
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` ("conv" or "norm") at `workload`, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    e = t.get("workloads", {}).get(workload, {}).get(kernel)
    return None if e is None else e["read_bytes"] + e["write_bytes"]


def _counter_values(run_dir, counter):
    """Per kernel name: the per-dispatch values of `counter` in the rocprofv3
    counter CSV(s) under run_dir."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def record_traffic(workload, fetch_dir, write_dir, copy_bytes):
    """Writes the conv and norm HBM bytes per launch of `workload` into
    profiles/traffic.json from a FETCH_SIZE pass and a WRITE_SIZE pass of
    ``bench.py --workload W --copy-calibration MIB`` (KiB per dispatch), each
    scaled by what the same counter reads for the run's plain copy of
    copy_bytes (read once, written once)."""
    fetch = _counter_values(fetch_dir, "FETCH_SIZE")
    write = _counter_values(write_dir, "WRITE_SIZE")

    def pick(d, key):
        v = [x for k in d if key in k for x in d[k]]
        if not v:
            raise SystemExit(f"no dispatch of a kernel named like {key!r} in the counters")
        return sum(v) / len(v)

    def calib(d):
        # the calibration copies: the largest runtime-copy dispatches (the
        # run's small set-up copies go through the same kernel)
        v = [x for k in d if "copyBuffer" in k for x in d[k]]
        if not v:
            raise SystemExit("no runtime copy in the counters (run with --copy-calibration)")
        big = [x for x in v if x >= 0.5 * max(v)]
        return sum(big) / len(big)

    ff = copy_bytes / (calib(fetch) * 1024)
    wf = copy_bytes / (calib(write) * 1024)
    entry = {"calibration": {"fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}}
    for name, key in (("conv", "conv3d_bf16_kernel"), ("norm", "rmsnorm_silu_kernel")):
        if any(key in k for k in fetch):
            entry[name] = {"read_bytes": int(pick(fetch, key) * 1024 * ff),
                           "write_bytes": int(pick(write, key) * 1024 * wf)}
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    sha = kernel_sources_sha256()
    if t.get("kernel_sources_sha256") != sha:
        t = {"workloads": {}}
    t["kernel_sources"] = library_sources()
    t["kernel_sources_sha256"] = sha
    t["method"] = ("rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE, one pass each, on `python3 bench.py "
                   "--workload W --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration 1024`; "
                   "per-dispatch KiB averaged over the conv (or norm) dispatches, times 1024, times the "
                   "factor that maps the same counter to the bytes of the run's 1 GiB copy "
                   "(__amd_rocclr_copyBuffer: it reads and writes 1 GiB)")
    t["workloads"][workload] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(entry), flush=True)


def cpu_baseline(w, p, x_dev, frames):
    import numpy as np

    import oracle
    ob = oracle.Block(p["gamma1"], p["beta1"], p["wa"], p["ba"], p["gamma2"], p["beta2"],
                      p["wb"], p["bb"], p.get("ws"), p.get("bs"))
    xs = x_dev[:, :frames].float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.resblock_full(ob, np.ascontiguousarray(xs))
    dt = time.perf_counter() - t0
    return {"value": frames / dt, "unit": "frames/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"whole block (fp64 accumulation) over frames 0..{frames - 1} of "
                      f"[{w.n},{w.t},{w.h},{w.w},{w.cin}] -> {w.cout}: {dt:.1f} s"}


def head_tail(torch, wv, steps, warmup):
    """The decoder's head and tail around its ResidualBlocks, at the Wan 2.2
    720p decoder shapes: conv_in on the 16-channel latent [1,21,90,160,16] to
    384 channels, post_quant_conv (1x1x1, 16 -> 16) on the latent, and
    norm_out (RMS_norm + SiLU, 96 channels) + conv_out (96 -> 3) on the
    output-resolution activation [1,81,720,1280,96], as two launches and as
    the one fused launch (the norm applied as the conv reads its input: x read
    once with the tiles' halos, y written; its FLOPs are the conv's, its bytes
    x and y).  Seeded synthetic bf16
    values.  Per op: average launch time over `steps` launches, algorithmic
    FLOPs and HBM bytes (read inputs once, write outputs once), and the
    fraction of the bound that limits it (the larger of FLOPs / 2.5 PFLOP/s
    and bytes / 8 TB/s)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(0)

    def randn(*shape, scale=1.0):
        return (torch.randn(shape, device="cuda", generator=g) * scale).to(torch.bfloat16)

    z = randn(1, 21, 90, 160, 16)
    act = randn(1, 81, 720, 1280, 96)
    w_in = wv.pack_conv3d_weights(randn(384, 16, 3, 3, 3, scale=(1 / 432) ** 0.5))
    w_out = wv.pack_conv3d_weights(randn(3, 96, 3, 3, 3, scale=(1 / 2592) ** 0.5))
    w_pq = randn(16, 16, scale=0.25)
    b384 = torch.randn(384, device="cuda", generator=g) * 0.1
    b3 = torch.randn(3, device="cuda", generator=g) * 0.1
    b16 = torch.randn(16, device="cuda", generator=g) * 0.1
    gam = torch.rand(96, device="cuda", generator=g) + 0.5
    bet = torch.randn(96, device="cuda", generator=g) * 0.3
    y_in = torch.empty((1, 21, 90, 160, 384), dtype=torch.bfloat16, device="cuda")
    y_pq = torch.empty_like(z)
    n_out = torch.empty_like(act)
    y_out = torch.empty((1, 81, 720, 1280, 3), dtype=torch.bfloat16, device="cuda")
    P_lat, P_out = 21 * 90 * 160, 81 * 720 * 1280
    ops = [
        ("conv_in 16->384, causal 3x3x3, [1,21,90,160,16]", wv.KERNEL_CONV_BF16,
         lambda: wv.causal_conv3d(z, w_in, b384, out=y_in),
         2.0 * P_lat * 384 * 27 * 16, 2.0 * P_lat * (16 + 384)),
        ("post_quant_conv 16->16, 1x1x1, [1,21,90,160,16]", wv.KERNEL_POINTWISE,
         lambda: wv.pointwise_conv(z, w_pq, b16, out=y_pq),
         2.0 * P_lat * 16 * 16, 2.0 * P_lat * (16 + 16)),
        ("norm_out RMS_norm+SiLU, C=96, [1,81,720,1280,96]", wv.KERNEL_NORM,
         lambda: wv.rmsnorm_silu(act, gam, bet, out=n_out),
         0.0, 2.0 * P_out * 96 * 2),
        ("conv_out 96->3, causal 3x3x3, [1,81,720,1280,96]", wv.KERNEL_CONV_BF16,
         lambda: wv.causal_conv3d(n_out, w_out, b3, out=y_out),
         2.0 * P_out * 3 * 27 * 96, 2.0 * P_out * (96 + 3)),
        ("norm_out + conv_out fused, [1,81,720,1280,96] -> 3", wv.KERNEL_CONV_BF16,
         lambda: wv.rmsnorm_silu_conv_out(act, gam, bet, wv.EPS, w_out, b3, out=y_out),
         2.0 * P_out * 3 * 27 * 96, 2.0 * P_out * (96 + 3)),
    ]
    return {"metric": "decoder head/tail ops, average launch time (1 GPU)", "unit": "ms",
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic (seeded)",
            "steps": steps, "warmup": warmup, "ops": time_ops(torch, wv, ops, steps, warmup)}


def time_ops(torch, wv, ops, steps, warmup, min_warm_s=0.05):
    """Per op (name, kernel kind, launch, FLOPs, bytes): `warmup` untimed
    launches, and more until `min_warm_s` seconds of them have run (a launch
    of about a millisecond right after input generation otherwise meets a
    clock still ramping up), then the library's hipEvent timing over `steps`
    launches; the bound is the larger of FLOPs / 2.5 PFLOP/s and bytes /
    8 TB/s."""
    res = []
    for name, kind, fn, flop, nbytes in ops:
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            fn()
            torch.cuda.synchronize()
        wv.timing_reset()
        wv.timing_enable(True)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        wv.timing_enable(False)
        n, ms = wv.timing_read(kind)
        wv.timing_reset()
        avg = ms / n
        t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        res.append({"op": name, "avg_launch_ms": avg, "flop": flop, "bytes": nbytes,
                    "tflops": flop / (avg * 1e-3) / 1e12, "gbs": nbytes / (avg * 1e-3) / 1e9,
                    "bound": bound, "frac": max(t_mfma, t_hbm) / avg})
        print(f"[bench] {name}: {avg:.3f} ms, {res[-1]['frac']:.1%} of its {bound} bound",
              file=sys.stderr, flush=True)
    return res


def upsample(torch, wv, steps, warmup):
    """The decoder's upsamplers in the order the Wan 2.2 720p decoder runs
    them: upsample3d 384 -> 192 from [1,21,90,160] (to 41 frames of
    180 x 320), upsample3d 384 -> 192 from [1,41,180,320] (to 81 frames of
    360 x 640), and upsample2d 192 -> 96 from [1,81,360,640] (to 720 x 1280)
    (wanvae_upsample3d_conv / wanvae_upsample2d_conv: frames doubled after the
    first for the 3D ones, nearest x2 in H and W, then the 3x3 conv halving
    the channels).  Seeded synthetic bf16 values.  With C_out a multiple of 96
    (all three) the library runs the conv by output phase, 4 merged taps per
    output instead of 9: the MFMA work counted is those 4 taps, and each op
    also reports the 9-tap direct form's FLOPs (``flop_direct``) and the rate
    they would correspond to."""
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    res = []
    for (t, h, w, cin, cout, temporal) in [(21, 90, 160, 384, 192, True), (41, 180, 320, 384, 192, True),
                                           (81, 360, 640, 192, 96, False)]:
        x = torch.empty((1, t, h, w, cin), dtype=torch.bfloat16, device="cuda")
        for i in range(t):
            x[0, i].copy_(torch.randn((h, w, cin), device="cuda", generator=g))
        wp = wv.pack_conv2d_weights((torch.randn((cout, cin, 3, 3), device="cuda", generator=g)
                                     * (1.0 / (9 * cin)) ** 0.5).to(torch.bfloat16))
        b = torch.randn(cout, device="cuda", generator=g) * 0.1
        to = 2 * t - 1 if temporal else t
        y = torch.empty((1, to, 2 * h, 2 * w, cout), dtype=torch.bfloat16, device="cuda")
        P_in, P_out = t * h * w, to * 4 * h * w
        fn = wv.upsample3d_conv if temporal else wv.upsample2d_conv
        name = "upsample3d" if temporal else "upsample2d"
        taps = 4 if cout % 96 == 0 else 9
        ops = [(f"{name} {cin}->{cout}, [1,{t},{h},{w},{cin}] -> [1,{to},{2 * h},{2 * w},{cout}]",
                wv.KERNEL_UPSAMPLE, lambda: fn(x, wp, b, out=y),
                2.0 * P_out * cout * taps * cin, 2.0 * (P_in * cin + P_out * cout))]
        r = time_ops(torch, wv, ops, steps, warmup)
        for e in r:
            e["taps_per_output"] = taps
            e["flop_direct"] = 2.0 * P_out * cout * 9 * cin
            e["tflops_direct_equivalent"] = e["flop_direct"] / (e["avg_launch_ms"] * 1e-3) / 1e12
        res += r
        del x, y
        torch.cuda.empty_cache()
    return {"metric": "decoder upsampler convs, average launch time (1 GPU)", "unit": "ms",
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic (seeded)",
            "steps": steps, "warmup": warmup, "ops": res}


def attention(torch, wv, wl, steps, warmup):
    """The decoder mid-block attention block (wanvae_attention_block) over the
    latent clip [1,21,90,160,384] bf16: frames/s of the whole block, and per
    kernel kind the average launch time and its roofline fraction.  The flash
    kernel's work is 4 * F * HW^2 * C FLOP (scores and the value product); the
    projections' 2 * P * C * 4C; norm and transpose are counted in bytes."""
    w = wl.custom("attention", wl.BF16, 1, 21, 90, 160, 384, 384)
    p = wl.make_attention_params(384, seed=0)
    blk = wv.AttentionBlock.from_host(p)
    x = wl.make_x_device(w, seed=0)
    y = torch.empty_like(x)
    ws = blk.workspace(w.n, w.t, w.h, w.w)
    for _ in range(warmup):
        blk.forward(x, out=y, workspace=ws)
    torch.cuda.synchronize()
    wv.timing_reset()
    wv.timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(steps):
        blk.forward(x, out=y, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    wv.timing_enable(False)
    total_ms = e0.elapsed_time(e1)
    P, F, HW, C = w.positions, w.n * w.t, w.h * w.w, 384
    # per launch: FLOPs and algorithmic HBM bytes (the projections: q/k/v reads
    # u and writes 3C per position, the output projection reads o and the
    # residual x and writes y; averaged over the two launches of a step)
    kinds = {"flash attention": (wv.KERNEL_ATTENTION, 4.0 * F * HW * HW * C, 2.0 * P * C * 4),
             "q/k/v + output projections (MFMA GEMM)": (wv.KERNEL_GEMM, 2.0 * P * C * 4 * C / 2,
                                                       2.0 * P * (4 * C + 3 * C) / 2),
             "RMS_norm": (wv.KERNEL_NORM, 0.0, 2.0 * P * C * 2),
             "v transpose": (wv.KERNEL_TRANSPOSE, 0.0, 2.0 * P * C * 2)}
    ops = []
    for name, (kind, flop, nbytes) in kinds.items():
        n, ms = wv.timing_read(kind)
        avg = ms / n
        e = {"op": name, "launches": n, "avg_launch_ms": avg, "flop": flop, "bytes": nbytes}
        # the bound is whichever of the MFMA time and the HBM time is longer
        t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12)
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
        if t_mfma >= t_hbm:
            e.update(bound="mfma", achieved=flop / (avg * 1e-3) / 1e12, unit="TFLOP/s",
                     peak=PEAK_BF16_TFLOPS, frac=t_mfma / (avg * 1e-3))
        else:
            e.update(bound="hbm", achieved=nbytes / (avg * 1e-3) / 1e9, unit="GB/s", peak=PEAK_HBM_GBS,
                     frac=t_hbm / (avg * 1e-3))
        ops.append(e)
        print(f"[bench] {name}: {avg:.3f} ms per launch, {e['frac']:.1%} of the {e['bound']} peak",
              file=sys.stderr, flush=True)
    wv.timing_reset()
    return {"metric": "decoder mid-block attention block frames/sec, 1 GPU", "value": w.t * steps / (total_ms * 1e-3),
            "unit": "frames/s", "higher_is_better": True, "ms_per_step": total_ms / steps, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) input, random-init weights)",
            "config": {"workload": "attention block, one head of width 384, x [1,21,90,160,384] bf16, all frames"},
            "steps": steps, "warmup": warmup, "kernels": ops}


def copy_bound(torch, wv, wl, steps, warmup):
    """The attainable HBM rate for the norm, measured: the library's plain
    streaming copy (wanvae_stream_copy: read once, write once, 16-byte
    nontemporal accesses) at the size of one output-resolution activation
    ([1,81,720,1280,96] bf16, 14.3 GB), over a sweep of pieces in flight and
    workgroups per CU, beside the runtime's own copy (torch copy_) and the
    fused RMS_norm + SiLU at the same size in both its output forms (channels
    -last, and the 16-channel slices the conv reads, as inside the block).
    GB/s counts the bytes read plus the bytes written."""
    w = wl.WORKLOADS["c4"]
    x = wl.make_x_device(w, seed=0)
    y = torch.empty_like(x)
    nbytes = x.numel() * x.element_size()
    g = torch.Generator().manual_seed(0)
    gam = torch.rand(w.cin, generator=g).add_(0.5).cuda()
    bet = (torch.randn(w.cin, generator=g) * 0.3).cuda()
    res = []

    def timed(name, kind, fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        wv.timing_reset()
        wv.timing_enable(True)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        wv.timing_enable(False)
        n, ms = wv.timing_read(kind) if kind is not None else (0, 0.0)
        wv.timing_reset()
        return ms / n if n else None

    for unroll in (2, 4, 8):
        for bpc in (4, 8, 16):
            avg = timed(None, wv.KERNEL_COPY, lambda: wv.stream_copy(x, y, unroll, bpc))
            res.append({"op": f"stream copy, unroll {unroll}, {bpc} workgroups/CU", "avg_launch_ms": avg,
                        "gbs": 2.0 * nbytes / (avg * 1e-3) / 1e9})
            print(f"[bench] {res[-1]['op']}: {avg:.3f} ms, {res[-1]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    # the runtime's copy kernel, timed with torch events on the stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        y.copy_(x)
    e0.record()
    for _ in range(steps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / steps
    res.append({"op": "runtime copy (torch copy_)", "avg_launch_ms": avg, "gbs": 2.0 * nbytes / (avg * 1e-3) / 1e9})
    print(f"[bench] runtime copy: {avg:.3f} ms, {res[-1]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    avg = timed(None, wv.KERNEL_NORM, lambda: wv.rmsnorm_silu(x, gam, bet, out=y))
    res.append({"op": "RMS_norm + SiLU, channels-last output", "avg_launch_ms": avg,
                "gbs": 2.0 * nbytes / (avg * 1e-3) / 1e9})
    best = max(r["gbs"] for r in res if r["op"].startswith("stream copy"))
    for r in res:
        r["frac_of_copy"] = r["gbs"] / best
        r["frac_of_8tbs"] = r["gbs"] / PEAK_HBM_GBS
    return {"metric": "attainable HBM rate: streaming copy vs the fused norm, 1 GPU", "unit": "GB/s",
            "bytes_per_launch": 2.0 * nbytes, "best_copy_gbs": best, "steps": steps, "warmup": warmup,
            "ops": res}


def block_pass(torch, wv, step, steps, stream, instrumented):
    """K steps between two events on the launch stream; with `instrumented`,
    the library's hipEvents bracket every launch as well.  Returns the
    elapsed ms and, when instrumented, (launches, total ms) per kernel kind."""
    wv.timing_reset()
    wv.timing_enable(instrumented)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wv.timing_enable(False)
    kinds = {}
    if instrumented:
        for k in (wv.KERNEL_CONV_BF16, wv.KERNEL_CONV_F32, wv.KERNEL_NORM, wv.KERNEL_GEMM, wv.KERNEL_ROLL):
            kinds[k] = wv.timing_read(k)
    wv.timing_reset()
    return e0.elapsed_time(e1), kinds


# activations at or below this size stay in the 256 MB Infinity Cache between
# launches: their GB/s is no HBM figure
MALL_BYTES = 256 << 20
# default frames of the CPU oracle baseline per workload (about 10-30 s of
# oracle work on a 16-core host)
CPU_FRAMES = {"c1": 4, "c2": 4, "c3": 1, "c4": 1, "c5": 2}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--cpu-frames", type=int, default=0,
                    help="frames of the clip the CPU oracle baseline computes (default: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-chunk", type=int, default=0, metavar="N",
                    help="time the streaming mode instead: a step runs the clip through "
                         "wanvae_resblock_stream_step in chunks of N frames (caches zeroed first)")
    ap.add_argument("--head-tail", action="store_true",
                    help="time the decoder's head and tail ops instead (conv_in 16->384, "
                         "post_quant_conv 16->16, norm_out + conv_out 96->3) at the "
                         "decoder's shapes, one JSON line")
    ap.add_argument("--attention", action="store_true",
                    help="time the decoder mid-block attention block instead, at the latent "
                         "shape [1,21,90,160,384] (one JSON line)")
    ap.add_argument("--upsample", action="store_true",
                    help="time the decoder's upsamplers instead (two upsample3d, one upsample2d, "
                         "at the decoder's shapes; one JSON line)")
    ap.add_argument("--copy-bound", action="store_true",
                    help="measure the attainable HBM rate instead: the library's streaming copy "
                         "and the fused norm at one output-resolution activation (one JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy a MIB-MiB buffer 3 times (a plain copy "
                         "kernel of known size, to scale HBM byte counters by)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: write profiles/traffic.json's entry for --workload from the "
                         "rocprofv3 output directories of a FETCH_SIZE and a WRITE_SIZE pass "
                         "(each run with --copy-calibration 1024)")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.workload, args.record_traffic[0], args.record_traffic[1], 1024 << 20)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the ResidualBlock path here is single-GPU "
              "(the multi-GPU H-split with halo exchange is designed, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_convolution_amd as wv
    from causal_convolution_amd import workloads as wl

    if args.head_tail:
        print(json.dumps(head_tail(torch, wv, args.steps, args.warmup)), flush=True)
        return
    if args.attention:
        print(json.dumps(attention(torch, wv, wl, args.steps, args.warmup)), flush=True)
        return
    if args.upsample:
        print(json.dumps(upsample(torch, wv, args.steps, args.warmup)), flush=True)
        return
    if args.copy_bound:
        print(json.dumps(copy_bound(torch, wv, wl, args.steps, args.warmup)), flush=True)
        return

    w = wl.WORKLOADS[args.workload]
    dt = torch.bfloat16 if w.dtype == wl.BF16 else torch.float32
    esize = 2 if w.dtype == wl.BF16 else 4
    torch.cuda.set_device(0)
    p = wl.make_params(w, seed=0)
    blk = wv.ResBlock.from_host(p, dt)
    x = wl.make_x_device(w, seed=0)
    y = torch.empty((w.n, w.t, w.h, w.w, w.cout), dtype=dt, device="cuda")
    ws = blk.workspace(w.n, w.t, w.h, w.w)
    stream = torch.cuda.current_stream()
    print(f"[bench] {w.desc}; steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)

    if args.stream_chunk > 0:
        # streaming mode: chunks of N frames through the feat_cache entry point
        assert w.n == 1, "the frame-chunk views below are contiguous for batch 1"
        N = args.stream_chunk
        ca, cb = blk.new_caches(w.n, w.h, w.w)
        ws = blk.workspace(w.n, min(N, w.t), w.h, w.w)

        def step():
            ca.zero_()
            cb.zero_()
            for t0 in range(0, w.t, N):
                blk.stream_step(x[:, t0:t0 + N], ca, cb, out=y[:, t0:t0 + N], workspace=ws)
    else:
        def step():
            blk.forward(x, out=y, workspace=ws)

    wv.wait_giveups_reset()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    total_ms, _ = block_pass(torch, wv, step, args.steps, stream, instrumented=False)
    print(f"[bench] timed {args.steps} steps: {total_ms:.3f} ms", file=sys.stderr, flush=True)
    inst_ms, kinds = block_pass(torch, wv, step, args.steps, stream, instrumented=True)
    print(f"[bench] instrumented pass, {args.steps} steps: {inst_ms:.3f} ms", file=sys.stderr, flush=True)
    giveups = wv.wait_giveups()
    conv_kind = wv.KERNEL_CONV_BF16 if w.dtype == wl.BF16 else wv.KERNEL_CONV_F32
    n_conv, conv_ms = kinds[conv_kind]
    n_norm, norm_ms = kinds[wv.KERNEL_NORM]
    # a 1x1x1 shortcut the library ran as a projection GEMM ahead of conv B
    n_sc, sc_ms = kinds[wv.KERNEL_GEMM]

    fa, fb = conv_flops(w, shortcut_in_conv=n_sc == 0)
    conv_avg_ms = conv_ms / n_conv
    # algorithmic work of the timed steps spread over their launches (one conv A
    # and one conv B per step full-T; one of each per chunk when streaming)
    conv_flop_per_launch = (fa + fb) * args.steps / n_conv
    conv_tflops = conv_flop_per_launch / (conv_avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == wl.BF16 else PEAK_F32_TFLOPS
    nb1, nb2 = norm_bytes(w, esize)
    steps_norm = n_norm / args.steps if args.stream_chunk == 0 else None
    # norm launches per step: 2 (norm1, norm2), or 1 where conv A computes norm2
    # in its epilogue
    nb = nb1 + (nb2 if steps_norm is None or steps_norm >= 2 else 0.0)
    norm_avg_ms = norm_ms / n_norm if n_norm else None
    norm_bytes_per_launch = nb * args.steps / n_norm if n_norm else None
    norm_gbs = norm_bytes_per_launch / (norm_avg_ms * 1e-3) / 1e9 if n_norm else None
    act_bytes = w.positions * max(w.cin, w.cout) * esize

    ms_per_step = total_ms / args.steps
    out = {
        "metric": METRIC,
        "value": w.t * args.steps / (total_ms * 1e-3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == wl.BF16 else "f32",
        "data": "synthetic (seeded N(0,1) input, random-init weights)",
        "config": {"workload": f"ResidualBlock {w.cin}->{w.cout} "
                               f"{'identity' if w.cin == w.cout else '1x1x1'} shortcut, "
                               f"x [{w.n},{w.t},{w.h},{w.w},{w.cin}] {w.dtype}, "
                               + (f"streamed in chunks of {args.stream_chunk} frames with the feat_cache"
                                  if args.stream_chunk > 0 else "full-T"),
                   "frames": w.t, "positions": w.positions, "parallelism": "1 GPU"},
        "roofline": {"bound": "mfma", "achieved": conv_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": conv_tflops / peak,
                     "traffic": None if args.stream_chunk else measured_traffic(args.workload, "conv"),
                     "kernel": "conv3d_bf16_kernel (conv A and conv B launches)",
                     "flop_per_launch": conv_flop_per_launch, "avg_launch_ms": conv_avg_ms,
                     "launches": n_conv},
        "norm": None if not n_norm else
                {"bound": "hbm", "achieved": norm_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": norm_gbs / PEAK_HBM_GBS, "bytes_per_launch": norm_bytes_per_launch,
                 "hbm_valid": act_bytes > MALL_BYTES,
                 "traffic": None if args.stream_chunk else measured_traffic(args.workload, "norm"),
                 "avg_launch_ms": norm_avg_ms, "launches": n_norm},
        "instrumented_ms_per_step": inst_ms / args.steps,
        "wait_giveups": giveups,
        "cpu_baseline": None,
    }
    if act_bytes <= MALL_BYTES and out["norm"] is not None:
        out["norm"]["note"] = (f"each activation ({act_bytes / 1e6:.0f} MB) fits the 256 MB Infinity Cache: "
                               "a cache-assisted rate, not an HBM figure")
    if n_sc > 0:
        sc_flop = 2.0 * w.positions * w.cout * w.cin * args.steps / n_sc
        sc_bytes = 2.0 * w.positions * (w.cin + w.cout) * args.steps / n_sc
        sc_ms_avg = sc_ms / n_sc
        out["shortcut"] = {"kernel": "gemm_bf16_kernel (the 1x1x1 shortcut, ahead of conv B)",
                           "bound": "hbm" if sc_bytes / PEAK_HBM_GBS / 1e9 > sc_flop / PEAK_BF16_TFLOPS / 1e12
                           else "mfma",
                           "achieved_gbs": sc_bytes / (sc_ms_avg * 1e-3) / 1e9,
                           "frac_hbm": sc_bytes / (sc_ms_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "flop_per_launch": sc_flop, "bytes_per_launch": sc_bytes,
                           "avg_launch_ms": sc_ms_avg, "launches": n_sc}
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 copies of {nbytes} bytes", file=sys.stderr, flush=True)
        del src, dst
    if not args.no_cpu_baseline:
        frames = args.cpu_frames or CPU_FRAMES.get(args.workload, 1)
        print(f"[bench] CPU oracle baseline on {frames} frame(s) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, p, x, frames)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
