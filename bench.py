#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 linear on one MI355X.

A step is one svdq_linear_forward (kernel 1: smoothing + 4-bit activation
quantization + X_hat L1; kernel 2: 4-bit GEMM + low-rank up-projection + bias)
over one batch of synthetic input already resident in HBM. The workload is
the FLUX-style MLP up-projection M=4608 tokens, K=3072 -> N=12288, rank 32,
MXFP4 (E2M1 + E8M0 per 32) -- the 4608x3072x12288 layer. `value` is effective
TOPS = 2*M*N*K / time per step (the low-rank flops are not counted).

Also measured in the same run: the GEMM kernel's average duration with HIP
events on the library's stream (roofline against the MXFP4 dense MFMA peak),
kernel 1's achieved HBM bandwidth, INT4 layers of the same family as a
secondary line, and the CPU oracle on a bounded sample of rows (baseline only).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SVDQuant W4A4 linear effective TOPS at 4608×3072×12288; % of MFMA peak"
PEAK_TFLOPS = {"mxfp4": 10100.0, "fp6": 10100.0, "i8": 5000.0}   # MI355X dense MFMA: FP4 and FP6
# 10.1 PF, INT8 5.0 POPS


def int4_gemm_mfma(M, N, cus):
    """The MFMA an INT4 layer's GEMM runs on: the tiled kernel's FP6 copies of
    the codes, or the few-token kernel's INT8 (the library's dispatch rule:
    at most 256 tokens, or 769 to 1024 unless the 32-channel blocks overfill
    one round of CUs by at most a quarter)."""
    nb = (N + 31) // 32
    small = M <= 256 or (768 < M <= 1024 and not (nb > cus and 4 * nb <= 5 * cus))
    return "i8" if small else "fp6"
PEAK_HBM_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "gemm_mxfp4_mlp_up_4608x3072x12288_counters.md")
GEMM_SOURCE = os.path.join(ROOT, "bit_svdquant_diffusion_amd", "csrc", "svdq_gemm_mxfp4.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_MARKS = [0]


def mark(args, torch, name):
    """With --layer-markers: one byte-fill kernel before a workload, so that a
    profiler trace attributes the dispatches after the k-th fill to the
    workload logged as marker k."""
    if not args.layer_markers:
        return
    _MARKS[0] += 1
    torch.full((4096,), _MARKS[0] % 256, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[marker {_MARKS[0]}] {name}")


def make_workload(spec, rotate, torch, S, synth, seed=0, packed=None):
    """Pack the layer with the library (randomized SVD) and replicate inputs,
    outputs, workspaces and packed weights `rotate` times in HBM. `packed`
    (layer, host) reuses another layer's packed weights."""
    import numpy as np
    t0 = time.time()
    lay = synth.make_layer(spec)
    if packed is None:
        ax = np.abs(lay.x).max(axis=0)
        layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
        host = S.pack_weights(layer, lay.w_lin, lay.bias, ax, seed=seed)
        log(f"  packed {spec.name} in {time.time() - t0:.1f}s")
    else:
        layer, host = packed
    x0 = torch.from_numpy(lay.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    sets = []
    wsb = S.workspace_bytes(layer, spec.M)
    for _ in range(rotate):
        dev = S.to_device(layer, host)
        sets.append(dict(
            dev=dev, x=x0.clone(),
            ws=torch.empty(wsb, dtype=torch.uint8, device="cuda"),
            y=torch.empty((spec.M, spec.N), dtype=torch.bfloat16, device="cuda")))
    return layer, host, lay, sets


def time_forward(layer, sets, steps, warmup, torch, S):
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        s = sets[i % len(sets)]
        S.linear_forward(layer, s["dev"], s["x"], y=s["y"], workspace=s["ws"], stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        s = sets[i % len(sets)]
        S.linear_forward(layer, s["dev"], s["x"], y=s["y"], workspace=s["ws"], stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def time_split(layer, sets, steps, warmup, torch, S):
    """Same steps as stage1 + gemm with events around each kernel (same stream)."""
    stream = torch.cuda.current_stream()
    M = sets[0]["x"].shape[0]
    for i in range(warmup):
        s = sets[i % len(sets)]
        S.stage1(layer, s["dev"], s["x"], s["ws"], stream=stream)
        S.gemm(layer, s["dev"], s["ws"], M, s["y"], stream=stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        s = sets[i % len(sets)]
        ev[i][0].record(stream)
        S.stage1(layer, s["dev"], s["x"], s["ws"], stream=stream)
        ev[i][1].record(stream)
        S.gemm(layer, s["dev"], s["ws"], M, s["y"], stream=stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    t2 = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    return t1, t2


def time_graph(calls, reps, torch):
    """Per-call GPU time of `calls` (each launches on the current stream),
    captured once into a HIP graph and replayed `reps` times: the launch
    cost of the host is out of the measurement."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for _ in range(max(3, reps)):   # untimed replays as many as the timed ones
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * len(calls))
    del g
    return ms


def stage1_bytes(spec):
    """Algorithmic HBM bytes of kernel 1: read X (bf16) and mu, L1; write codes, scales, Z."""
    r32 = (spec.rank + 31) // 32 * 32
    scale = spec.M * spec.K // 64 * 4 if spec.fmt == "int4" else spec.M * spec.K // 32
    return (spec.M * spec.K * 2 + spec.K * 4 + spec.K * r32 * 2 + spec.M * spec.K // 2 + scale
            + spec.M * r32 * 2)


def gemm_bytes(spec):
    """Algorithmic HBM bytes of kernel 2: read codes + scales of X and W, Z, L2, bias; write Y."""
    r32 = (spec.rank + 31) // 32 * 32
    g = 64 if spec.fmt == "int4" else 32
    sbytes = 4 if spec.fmt == "int4" else 1
    return ((spec.M + spec.N) * spec.K // 2 + (spec.M + spec.N) * spec.K // g * sbytes
            + (spec.M + spec.N) * r32 * 2 + spec.N * 2 + spec.M * spec.N * 2)


def traffic_from_profile():
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken on the current GEMM source (sha256 recorded in the summary)."""
    try:
        txt = open(PROFILE_COUNTERS).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    m_sha = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_sha and m_b) or m_sha.group(1) != src:
        return None
    return float(m_b.group(1))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_info():
    """(vendor, threads) of the BLAS numpy uses, from threadpoolctl when present."""
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                return f"{p.get('internal_api')} {p.get('version') or ''}".strip(), p.get("num_threads")
    except Exception:
        pass
    return "unknown", None


def cpu_baseline(layer, host, lay, spec, budget_s):
    """The oracle's forward on a bounded sample of the same workload's rows,
    with the same packed weights (logical values), on all of the host cores
    this process may use; the median of three timed runs of that sample."""
    import contextlib
    import numpy as np
    from oracle import svdq_oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    import bit_svdquant_diffusion_amd as S
    cores = len(os.sched_getaffinity(0))
    u = S.unpack_weights(layer, host)
    packed = dict(fmt=spec.fmt, mu=u["mu"], l1=O.bf16_from_bits(u["l1"]),
                  l2=O.bf16_from_bits(u["l2"]), bias=O.bf16_from_bits(u["bias"]),
                  qw=u["codes"] if spec.fmt == "int4" else u["codes"].astype(np.uint8),
                  sw=u["scales"])
    ctx = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        vendor, threads = _blas_info()
        # size the sample so that one run takes about a third of the budget
        rows = 64
        while True:
            t0 = time.perf_counter()
            O.forward(packed, lay.x[:rows])
            t = time.perf_counter() - t0
            if t >= budget_s / 6 or rows >= spec.M:
                break
            rows = int(min(spec.M, max(2 * rows, rows * 0.3 * budget_s / max(t, 1e-3)) // 64 * 64))
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.forward(packed, lay.x[:rows])
            times.append(time.perf_counter() - t0)
    t = sorted(times)[1]
    tops = 2.0 * rows * spec.N * spec.K / t / 1e12
    return dict(value=round(tops, 6), unit="TOPS", cores=cores, kind="oracle",
                sample=f"{rows} of {spec.M} token rows of the same layer ({spec.M}x{spec.K}->{spec.N}, "
                       f"r{spec.rank}, {spec.fmt}); oracle forward (NumPy float64), median of 3 runs "
                       f"({', '.join(f'{x:.2f}' for x in times)} s); pack excluded",
                cpu_model=_cpu_model(), blas=vendor, blas_threads=threads)


def measured_peaks(torch, S, reps=5):
    """Measured ceilings of this GPU in the same process: the MFMA-only loop
    of each matrix instruction the GEMMs use (random and constant operand
    bits) and a 2 GiB device copy, each the median of `reps` event-timed runs."""
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            v = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return v, sorted(ts)[len(ts) // 2]

    out = {}
    for kind, iters in (("mxfp4", 20000), ("int8", 10000), ("bf16", 10000)):
        for const in (False, True):
            fl, t = timed(lambda: S.measure_mfma_peak(kind, iters, constant=const, stream=stream))
            out[f"{kind}_{'constant' if const else 'random'}_tflops"] = round(fl / t / 1e12, 1)
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    _, t = timed(lambda: S.measure_copy(src, dst, stream=stream))
    out["copy_gbs"] = round(2 * n / t / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def settle(layer, sets, torch, S, seconds=0.5):
    """Run forwards untimed for a fixed time before the warm-up steps: after
    the host-side pack the GPU has been idle and its clocks take tens of
    milliseconds to come back up."""
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            s = sets[i % len(sets)]
            S.linear_forward(layer, s["dev"], s["x"], y=s["y"], workspace=s["ws"], stream=stream)
            i += 1
        torch.cuda.synchronize()
    return i


def awq_bytes(spec):
    """Algorithmic HBM bytes of one W4A16 launch: codes, scales and zero
    points, inv_s, bias, x in and y out."""
    return (spec.N * spec.K // 2 + spec.N * (spec.K // 128) * 5 + spec.K * 4 + spec.N * 2
            + spec.M * spec.K * 2 + spec.M * spec.N * 2)


def bench_awq(args, torch, S, synth):
    """The AWQ-style W4A16 layers (FLUX modulation and final-norm shapes):
    library pack with the alpha search on 32 held-out calibration rows, then
    GPU time per call from graph replays over 16 weight sets (far more bytes
    than the 256 MB MALL), against 8 TB/s."""
    import numpy as np
    rows = []
    for sp in synth.awq_layers():
        mark(args, torch, f"awq {sp.name}")
        lay = synth.make_layer(sp)
        t0 = time.time()
        host, alpha, _ = S.awq_pack(lay.w_lin, lay.bias, synth.calibration_rows(sp, 32))
        log(f"  packed {sp.name} (alpha {alpha}) in {time.time() - t0:.1f}s")
        x = torch.from_numpy(lay.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        sets = [dict(dev=S.awq_to_device(host), y=torch.empty((sp.M, sp.N), dtype=torch.bfloat16, device="cuda"))
                for _ in range(16)]
        calls = [lambda s=s: S.awq_forward(sp.K, sp.N, s["dev"], x, y=s["y"]) for s in sets]
        ms = time_graph(calls, max(8, args.steps // 4), torch)
        b = awq_bytes(sp)
        gbs = b / (ms * 1e-3) / 1e9
        rows.append({"workload": sp.name, "M": sp.M, "K": sp.K, "N": sp.N, "alpha": alpha, "us": round(ms * 1e3, 2),
                     "hbm_algorithmic_bytes": b, "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        log(f"awq {sp.name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s)")
        del sets
        torch.cuda.empty_cache()
    return {"workload": "AWQ-style W4A16 linears, FLUX modulation and final-norm shapes, batch 2 and 16",
            "kernel": "svdq::awq_kernel", "bound": "hbm", "layers": rows}


def bench_c4(args, torch, S, synth):
    """Config 4: a FLUX double-stream block's linears at batch 2, 1024^2 (image
    M=8192, text M=1024) and the decode-like M=64, 256 runs of the same four
    shapes, which reuse the text stream's packed weights. Per layer: forward
    time (GPU time from HIP graph replays, with the rate of eager launches
    beside it), effective TOPS and, for the small-M runs, algorithmic HBM
    bytes per second against 8 TB/s. Small-M runs rotate 16 weight sets so
    that the 256 MB MALL cannot hold them."""
    packs, rows = {}, []
    steps = max(10, args.steps // 5)
    for li, sp in enumerate(synth.config_layers(4)):
        mark(args, torch, f"c4 {sp.name}")
        owner = sp.stream or sp.name
        rot = 16 if sp.M <= 256 else 2
        layer, host, _, sets = make_workload(sp, rot, torch, S, synth, packed=packs.get(owner))
        packs[owner] = (layer, host)
        ms_eager, _ = time_forward(layer, sets, steps, max(20, args.warmup // 10), torch, S)
        # GPU time per call from graph replays of one call per buffer set
        # (the few-token layers launch faster than the host can issue them)
        reps = max(4, steps // len(sets))
        fwd = [lambda s=s: S.linear_forward(layer, s["dev"], s["x"], y=s["y"], workspace=s["ws"]) for s in sets]
        s1 = [lambda s=s: S.stage1(layer, s["dev"], s["x"], s["ws"]) for s in sets]
        gm = [lambda s=s: S.gemm(layer, s["dev"], s["ws"], sp.M, s["y"]) for s in sets]
        ms = time_graph(fwd, reps, torch)
        a1 = time_graph(s1, reps, torch)
        a2 = time_graph(gm, reps, torch)
        del sets
        torch.cuda.empty_cache()
        fl = 2.0 * sp.M * sp.N * sp.K
        hb = stage1_bytes(sp) + gemm_bytes(sp)
        t = fl / (ms * 1e-3) / 1e12
        mf = int4_gemm_mfma(sp.M, sp.N, torch.cuda.get_device_properties(0).multi_processor_count)
        gbs = hb / (ms * 1e-3) / 1e9
        rows.append({"workload": sp.name, "M": sp.M, "K": sp.K, "N": sp.N, "rank": sp.rank, "format": sp.fmt,
                     "us": round(ms * 1e3, 2), "us_eager_launches": round(ms_eager * 1e3, 2),
                     "effective_tops": round(t, 2), "gemm_mfma": mf,
                     "pct_of_mfma_peak": round(100 * t / PEAK_TFLOPS[mf], 2),
                     "hbm_algorithmic_bytes": hb, "hbm_gbs": round(gbs, 1),
                     "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                     "stage1_us": round(a1 * 1e3, 2), "gemm_us": round(a2 * 1e3, 2)})
        log(f"c4 {sp.name}: {ms * 1e3:.1f} us (eager {ms_eager * 1e3:.1f}), {t:.1f} TOPS, {gbs:.0f} GB/s "
            f"(stage1 {a1 * 1e3:.1f} us, gemm {a2 * 1e3:.1f} us)")
    block = [r for r in rows if r["workload"].startswith(("img_", "txt_"))]
    bus = sum(r["us"] for r in block)
    bops = sum(2.0 * r["M"] * r["N"] * r["K"] for r in block)
    return {"workload": "FLUX double-stream block linears, batch 2, 1024^2, INT4 g64, r32",
            "layers": rows, "block_us": round(bus, 1),
            "block_effective_tops": round(bops / (bus * 1e-6) / 1e12, 2)}


def bench_mlp(args, torch, S, synth):
    """The image stream's MLP of a FLUX double-stream block (3072 -> 12288 ->
    3072, rank 32, INT4) as one svdq_mlp_forward: fused (the up GEMM's
    epilogue emits the down layer's codes, scales and partial Z; the hidden
    activation never reaches HBM) against the composition (up, GELU kernel,
    down), at batch 2 (8192 tokens) and at one image with its text (4608).
    GPU time per call from graph replays over 2 buffer sets."""
    import numpy as np
    by = {s.name: s for s in synth.config_layers(4, small_m=False)}
    su, sd = by["img_up"], by["img_down"]
    lay_u, lay_d = synth.make_layer(su), synth.make_layer(sd)
    t0 = time.time()
    lu, ld = S.Layer(su.K, su.N, su.rank, su.fmt), S.Layer(sd.K, sd.N, sd.rank, sd.fmt)
    hu = S.pack_weights(lu, lay_u.w_lin, lay_u.bias, np.abs(lay_u.x).max(axis=0))
    hd = S.pack_weights(ld, lay_d.w_lin, lay_d.bias, np.abs(lay_d.x).max(axis=0))
    log(f"  packed the MLP pair in {time.time() - t0:.1f}s")
    rows = []
    for M in (8192, 4608):
        mark(args, torch, f"mlp M={M} (fused, then composition)")
        x = torch.from_numpy(lay_u.x_bits[:M].view(np.int16)).cuda().view(torch.bfloat16)
        wsb = S.mlp_workspace_bytes(lu, ld, M)[0]
        sets = [dict(du=S.to_device(lu, hu), dd=S.to_device(ld, hd), ws=torch.empty(wsb, dtype=torch.uint8, device="cuda"),
                     y=torch.empty((M, sd.N), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
        res = {}
        for mode, name in ((S.MLP_AUTO, "fused"), (S.MLP_UNFUSED, "composition")):
            calls = [lambda s=s, mode=mode: S.mlp_forward(lu, s["du"], ld, s["dd"], x, y=s["y"], workspace=s["ws"],
                                                          mode=mode) for s in sets]
            res[name] = time_graph(calls, max(10, args.steps // 5), torch)
        fl = 2.0 * M * (su.K * su.N + sd.K * sd.N)
        hid = M * su.N * 2
        zpart = (su.N // 256) * M * 32 * 4
        rows.append({"M": M, "format": "int4", "fused": S.mlp_fused(lu, ld, M), "us_fused": round(res["fused"] * 1e3, 1),
                     "us_composition": round(res["composition"] * 1e3, 1),
                     "speedup": round(res["composition"] / res["fused"], 3),
                     "effective_tops_fused": round(fl / (res["fused"] * 1e-3) / 1e12, 1),
                     "composition_hidden_bytes": 4 * hid, "fused_partial_z_bytes": 2 * zpart})
        log(f"mlp M={M}: fused {res['fused'] * 1e3:.1f} us, composition {res['composition'] * 1e3:.1f} us "
            f"({res['composition'] / res['fused']:.3f}x)")
        del sets
        torch.cuda.empty_cache()
    # the MXFP4 pair at 4608 tokens: the headline layer and its down layer
    su2 = synth.config_layers(2)[0]
    sd2 = synth.LayerSpec("mlp_down_fp4", su2.M, su2.N, su2.K, 32, "mxfp4", 3, x_kind="gelu",
                          x_outlier_frac=0.005, x_outlier_scale=30.0, w_outlier_frac=0.0)
    lu2, ld2 = S.Layer(su2.K, su2.N, 32, "mxfp4"), S.Layer(sd2.K, sd2.N, 32, "mxfp4")
    lay_u2, lay_d2 = synth.make_layer(su2), synth.make_layer(sd2)
    hu2 = S.pack_weights(lu2, lay_u2.w_lin, lay_u2.bias, np.abs(lay_u2.x).max(axis=0))
    hd2 = S.pack_weights(ld2, lay_d2.w_lin, lay_d2.bias, np.abs(lay_d2.x).max(axis=0))
    M = su2.M
    mark(args, torch, f"mlp mxfp4 M={M} (fused, then composition)")
    x = torch.from_numpy(lay_u2.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    wsb = S.mlp_workspace_bytes(lu2, ld2, M)[0]
    sets = [dict(du=S.to_device(lu2, hu2), dd=S.to_device(ld2, hd2), ws=torch.empty(wsb, dtype=torch.uint8, device="cuda"),
                 y=torch.empty((M, sd2.N), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    res = {}
    for mode, name in ((S.MLP_AUTO, "fused"), (S.MLP_UNFUSED, "composition")):
        calls = [lambda s=s, mode=mode: S.mlp_forward(lu2, s["du"], ld2, s["dd"], x, y=s["y"], workspace=s["ws"],
                                                      mode=mode) for s in sets]
        res[name] = time_graph(calls, max(10, args.steps // 5), torch)
    fl = 2.0 * M * (su2.K * su2.N + sd2.K * sd2.N)
    rows.append({"M": M, "format": "mxfp4", "fused": S.mlp_fused(lu2, ld2, M),
                 "us_fused": round(res["fused"] * 1e3, 1), "us_composition": round(res["composition"] * 1e3, 1),
                 "speedup": round(res["composition"] / res["fused"], 3),
                 "effective_tops_fused": round(fl / (res["fused"] * 1e-3) / 1e12, 1),
                 "composition_hidden_bytes": 4 * M * su2.N * 2, "fused_partial_z_bytes": 2 * (su2.N // 384) * M * 32 * 4})
    log(f"mlp mxfp4 M={M}: fused {res['fused'] * 1e3:.1f} us, composition {res['composition'] * 1e3:.1f} us "
        f"({res['composition'] / res['fused']:.3f}x)")
    del sets
    torch.cuda.empty_cache()
    return {"workload": "FLUX MLP 3072 -> 12288 -> 3072 (GELU), r32: the double-stream image pair in INT4 g64 "
                        "(8192 and 4608 tokens) and the headline MXFP4 layer with its down layer (4608 tokens)",
            "note": "the composition moves the bf16 hidden activation four times (the up GEMM writes it, "
                    "the GELU kernel reads and rewrites it, the down layer's kernel 1 reads it); the fused "
                    "path writes and reads fp32 partial Z per 256 hidden channels instead",
            "runs": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first: clocks and caches take tens of milliseconds to settle")
    ap.add_argument("--rotate", type=int, default=4, help="distinct buffer sets cycled (defeats the 256 MB MALL)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-c4", action="store_true", help="skip the FLUX block's linears (config 4)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA and copy ceilings")
    ap.add_argument("--no-awq", action="store_true", help="skip the W4A16 (AWQ-style) layers")
    ap.add_argument("--no-mlp", action="store_true", help="skip the fused MLP pair")
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the half second of untimed forwards before the warm-up (profiler runs)")
    ap.add_argument("--layer-markers", action="store_true",
                    help="launch one byte-fill kernel before each workload (boundaries in profiler traces)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (reference kernel for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the layer shards over tokens with no exchange, see the "
              f"design notes. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_svdquant_diffusion_amd as S
    from bit_svdquant_diffusion_amd import synth

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    S.lib()
    log(f"device: {torch.cuda.get_device_name(0)}")

    spec = synth.config_layers(2)[0]          # 4608 x 3072 -> 12288, r32, MXFP4
    mark(args, torch, f"headline {spec.name}")
    layer, host, lay, sets = make_workload(spec, args.rotate, torch, S, synth)
    flops = 2.0 * spec.M * spec.N * spec.K

    nsettle = 0 if args.no_settle else settle(layer, sets, torch, S)
    ms, wall_ms = time_forward(layer, sets, args.steps, args.warmup, torch, S)
    tops = flops / (ms * 1e-3) / 1e12
    log(f"forward: {ms * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f} us), {tops:.1f} effective TOPS")
    t1, t2 = time_split(layer, sets, args.steps, args.warmup, torch, S)
    gemm_tflops = flops / (t2 * 1e-3) / 1e12
    s1_gbs = stage1_bytes(spec) / (t1 * 1e-3) / 1e9
    log(f"stage1 {t1 * 1e3:.1f} us ({s1_gbs:.0f} GB/s), gemm {t2 * 1e3:.1f} us ({gemm_tflops:.1f} TFLOP/s)")

    if args.copy_calib_mb:
        src = torch.empty(args.copy_calib_mb << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    traffic = traffic_from_profile()
    peaks = None if args.no_peaks else measured_peaks(torch, S)
    if peaks:
        log(f"measured peaks: {peaks}")
    out = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "FLUX-style MLP up-projection, MXFP4 SVDQuant W4A4 linear",
                   "M": spec.M, "K": spec.K, "N": spec.N, "rank": spec.rank, "format": spec.fmt,
                   "group": 32, "io": "bf16", "parallelism": "single GPU"},
        "pct_of_mfma_peak": round(100.0 * tops / PEAK_TFLOPS["mxfp4"], 2),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_TFLOPS["mxfp4"],
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_TFLOPS["mxfp4"], 4),
                     "traffic": traffic, "kernel": "svdq::gemm_mxfp4_kernel (persistent, 192x384 tiles)",
                     "kernel_avg_us": round(t2 * 1e3, 2), "algorithmic_bytes": gemm_bytes(spec),
                     "measured_peak": peaks["mxfp4_random_tflops"] if peaks else None,
                     "frac_of_measured": round(gemm_tflops / peaks["mxfp4_random_tflops"], 4) if peaks else None},
        "stage1": {"kernel": "stage1_kernel<MXFP4>", "avg_us": round(t1 * 1e3, 2), "bound": "hbm",
                   "achieved": round(s1_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(s1_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": stage1_bytes(spec),
                   "measured_peak": peaks["copy_gbs"] if peaks else None,
                   "frac_of_measured": round(s1_gbs / peaks["copy_gbs"], 4) if peaks else None},
        "settle_steps": nsettle,
    }
    if peaks:
        out["measured_peaks"] = peaks
    if not args.no_secondary:
        sec = []
        for idx in (3, 1):
            sp = synth.config_layers(idx)[0]
            mark(args, torch, f"secondary {sp.name}")
            del sets
            torch.cuda.empty_cache()
            l2, _, _, sets = make_workload(sp, args.rotate, torch, S, synth)
            ms2, _ = time_forward(l2, sets, max(10, args.steps // 2), args.warmup, torch, S)
            a1, a2 = time_split(l2, sets, max(10, args.steps // 2), args.warmup, torch, S)
            fl = 2.0 * sp.M * sp.N * sp.K
            t = fl / (ms2 * 1e-3) / 1e12
            sec.append({"workload": sp.name, "M": sp.M, "K": sp.K, "N": sp.N, "rank": sp.rank,
                        "format": sp.fmt, "ms_per_step": round(ms2, 6), "effective_tops": round(t, 2),
                        "gemm_mfma": "fp6", "pct_of_mfma_peak": round(100 * t / PEAK_TFLOPS["fp6"], 2),
                        "stage1_us": round(a1 * 1e3, 2), "gemm_us": round(a2 * 1e3, 2)})
            log(f"{sp.name}: {ms2 * 1e3:.1f} us/step, {t:.1f} TOPS (stage1 {a1*1e3:.1f} us, gemm {a2*1e3:.1f} us)")
        out["secondary"] = sec
    if not args.no_c4:
        out["c4"] = bench_c4(args, torch, S, synth)
    if not args.no_mlp:
        out["mlp"] = bench_mlp(args, torch, S, synth)
    if not args.no_awq:
        out["awq"] = bench_awq(args, torch, S, synth)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(layer, host, lay, spec, args.cpu_budget)
        log(f"  {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
