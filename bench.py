"""Benchmark of one Muon optimizer step on one MI355X.

A step is one ``muon_step`` call over every matrix of the workload: momentum,
Frobenius normalisation, five Newton-Schulz iterations on bf16 matrix cores
and the parameter update.  Inputs are synthetic (low rank plus noise, drawn
on the GPU) and resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line on stdout.  Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
# Sources of the kernel whose counters the traffic record holds.
TRAFFIC_SOURCES = ("gemm32_kernels.hip", "muon_internal.h")
METRIC = "Muon optimizer steps/sec on 1.5B-shaped hidden params; NS5 TFLOP/s % of bf16 peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ns_flops(shapes, kind):
    """Algorithmic flops of one Newton-Schulz iteration (symmetry exploited).

    Per matrix with Gram side m and long side n: Gram m^2 n (upper half of
    2 m^2 n), polynomial m^3 (upper half of 2 m^3), BX 2 m^2 n."""
    tot = 0.0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        if kind == "gram":
            tot += m * m * n
        elif kind == "poly":
            tot += m ** 3
        elif kind == "bx":
            tot += 2.0 * m * m * n
    return tot


def _code_only(text):
    """Source text without comments, blank lines or indentation changes:
    what the compiler sees, so a comment edit does not void a record."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = (" ".join(ln.split()) for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash(names):
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "matrix_muon_step_amd", "csrc", nm), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_files, workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(kernel_files):
        return None
    return round(rec.get("bytes_per_launch"))


BX_KERNEL_RE = {
    # (Gram-side tile rows, long-side tile columns) -> rocprofv3 kernel-name pattern of the BX launch
    (160, 256): r"ns_gemm32_kernel<[^<]*G32<160, 256, 1, 4, 3>, 2>",
    (256, 256): r"ns_gemm32_kernel<[^<]*G32<256, 256, 2, 4, 4>, 2>",
    (320, 256): r"ns_gemm32_kernel<[^<]*G32<320, 256, 2, 4, 4>, 2>",
}
BX_KERNEL_NAME = {(160, 256): "W160", (256, 256): "G256", (320, 256): "W320"}
CALIB_RE = r"copy_probe_kernel"


def read_counter_csv(path, counter):
    """{kernel name: [value per dispatch]} of one counter from a rocprofv3
    counter_collection.csv."""
    import csv
    per = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            per.setdefault(row["Kernel_Name"], {}).setdefault(row["Dispatch_Id"], 0.0)
            per[row["Kernel_Name"]][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def record_traffic(workload, fetch_csv, write_csv, calib_bytes):
    """HBM bytes per launch of the dominant kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the library's plain copy kernel, which reads and
    writes calib_bytes.  Writes profiles/traffic_<workload>.json."""
    import re
    import statistics
    import matrix_muon_step_amd as mm
    w = synth.WORKLOADS[workload]
    shapes = [(s.rows, s.cols) for s in w.matrices]
    cfgs = sorted({(p["bx_tile_rows"], p["bx_tile_cols"]) for p in mm.muon_plan_query(shapes)[1] if p["tile"]})
    assert len(cfgs) == 1 and cfgs[0] in BX_KERNEL_RE, cfgs
    pat = re.compile(BX_KERNEL_RE[cfgs[0]])
    rec = {"workload": workload, "kernel_pattern": BX_KERNEL_RE[cfgs[0]],
           "source_hash": source_hash(TRAFFIC_SOURCES)}
    for name, path in (("fetch", fetch_csv), ("write", write_csv)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        per = read_counter_csv(path, counter)
        cal = [v for k, vs in per.items() if re.search(CALIB_RE, k) for v in vs]
        cal = cal[:1]  # the calibration copy is the first copy-kernel dispatch
        bx = [v for k, vs in per.items() if pat.search(k) for v in vs]
        assert cal and bx, (name, list(per))
        factor = calib_bytes / (max(cal) * 1024.0)
        rec[f"{name}_kib_per_launch_raw"] = statistics.mean(bx)
        rec[f"{name}_calibration_kib"] = max(cal)
        rec[f"{name}_factor"] = round(factor, 4)
        rec[f"{name}_bytes_per_launch"] = statistics.mean(bx) * 1024.0 * factor
        rec[f"{name}_launches"] = len(bx)
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def cpu_info():
    """Host CPU model, logical CPU count and the BLAS numpy runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        import threadpoolctl
        infos = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
            threads = max(int(i.get("num_threads", 1)) for i in infos)
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas": blas, "blas_threads": threads}


def cpu_baseline(w, budget_s=20.0):
    """The oracle on the host cores, on a bounded sample of the workload's
    matrices (whole layers, in order), scaled to one full step."""
    from oracle import muon_oracle
    info = cpu_info()
    per_layer = 6 if len(w.matrices) % 6 == 0 else 1
    t_used = 0.0
    done = 0
    params_done = 0
    while done < len(w.matrices) and t_used < budget_s:
        for i in range(done, min(done + per_layer, len(w.matrices))):
            h = synth.numpy_matrix(w, i, 0)
            g = synth.gradient_as_f64(h["G"], w.g_dtype)
            t0 = time.perf_counter()
            muon_oracle.muon_step(h["W0"], g, h["B0"], w.mu, w.lr, w.scale, 5)
            t_used += time.perf_counter() - t0
            params_done += w.matrices[i].rows * w.matrices[i].cols
        done = min(done + per_layer, len(w.matrices))
    step_s = t_used * (w.n_params / params_done)
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": int(info["blas_threads"] or 1), "kind": "oracle",
            "sample": f"first {done} of {len(w.matrices)} matrices ({params_done / 1e6:.1f}M of "
                      f"{w.n_params / 1e6:.1f}M params), one fp64 Muon step each, "
                      f"{t_used:.1f} s, scaled by parameter count (extrapolated)",
            "seconds_measured": round(t_used, 3), **info}


def copy_ceiling_gbps(dev, nbytes=2**30, reps=10):
    """Measured HBM ceiling of the bandwidth-bound stages: the fastest variant
    of the library's streaming copy kernel (read + write nbytes), HIP events
    on the launch stream."""
    import torch
    import matrix_muon_step_amd as mm

    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    best = None
    for v in range(mm.MUON_COPY_PROBE_VARIANTS):
        mm.muon_copy_probe(src, dst, v)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            mm.muon_copy_probe(src, dst, v)
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = 2.0 * nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, v)
    ok = bool(torch.equal(src, dst))
    del src, dst
    if not ok:
        raise RuntimeError("copy probe produced a wrong copy")
    return best


# Steps timed per workload in the default run (the headline uses --steps).
DEFAULT_STEPS = {"single256": 200, "gpt2s_fc_10step": 100, "gpt2_small": 50, "gpt2_xl_1p5b": 20, "moe_share": 10}
LATENCY_BOUND = ("single256", "gpt2s_fc_10step")


def make_inputs(w, dev, gen):
    import torch
    mats = []
    for i in range(len(w.matrices)):
        t = synth.torch_matrix(w, i, 0, dev, generator=gen)
        mats.append((t["W0"], t["G"], t["B0"], w.scale))
    # gpt2s_fc_10step: consecutive steps of one matrix, each with a fresh gradient
    grads = None
    if w.steps > 1:
        grads = [[synth.torch_matrix(w, i, t, dev, generator=gen)["G"] for i in range(len(w.matrices))]
                 for t in range(w.steps)]
    torch.cuda.synchronize()
    return mats, grads


def bench_workload(w, steps, warmup, ns_steps, dev, headline, diag_steps=0, copy_ceiling=None):
    """Times `steps` muon_step calls of workload w (profiling off), then a
    separate profiled pass for the per-stage breakdown and the dominant
    kernel's launch time.  Returns the workload's record."""
    import torch
    import matrix_muon_step_amd as mm

    shapes = [(s.rows, s.cols) for s in w.matrices]
    gen = torch.Generator(device=dev)
    gen.manual_seed(20240 + w.wid)
    mats, grads = make_inputs(w, dev, gen)
    ws_bytes = mm.muon_workspace_bytes(mats, mu=w.mu, lr=w.lr, ns_steps=ns_steps)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: {len(shapes)} matrices, {w.n_params / 1e9:.4f}B params, "
        f"workspace {ws_bytes / 2**30:.2f} GiB")
    k = [0]

    def step():
        cur = mats
        if grads is not None:
            g = grads[k[0] % len(grads)]
            cur = [(W, g[i], B, s) for i, (W, _, B, s) in enumerate(mats)]
        k[0] += 1
        mm.muon_step(cur, mu=w.mu, lr=w.lr, ns_steps=ns_steps, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / steps
    log(f"[bench] {w.name}: timed {steps} steps, {ms_per_step:.4f} ms/step "
        f"(host wall {wall / steps * 1e3:.4f} ms/step)")

    # ---- profiled pass: HIP events around every launch, on the launch stream
    psteps = max(1, min(steps, 5))
    mm.muon_profile_read()
    mm.muon_profile_enable(True)
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(psteps):
        step()
    p1.record(stream)
    torch.cuda.synchronize()
    mm.muon_profile_enable(False)
    prof = mm.muon_profile_read()
    prof_ms = p0.elapsed_time(p1) / psteps
    log(f"[bench] {w.name}: profiled {psteps} steps, {prof_ms:.4f} ms/step")

    big = [s for s in shapes if min(s) > 64]
    stage_ms = {kk: v[0] / psteps for kk, v in prof.items()}
    fl = {kk: ns_flops(big, kk) * ns_steps for kk in ("gram", "poly", "bx")}
    ns_ms = stage_ms["gram"] + stage_ms["poly"] + stage_ms["bx"] + stage_ms["bx_update"]
    ns_alg = fl["gram"] + fl["poly"] + fl["bx"]
    ns_tflops = ns_alg / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None
    dense_eq = sum(4.0 * min(s) ** 2 * max(s) + 2.0 * min(s) ** 3 for s in big) * ns_steps
    bx_iters = (ns_steps - 1) * psteps
    bx_avg_ms = prof["bx"][0] / bx_iters if bx_iters and prof["bx"][1] else None
    bx_flops_per_launch = ns_flops(big, "bx")
    bx_tflops = bx_flops_per_launch / (bx_avg_ms * 1e-3) / 1e12 if bx_avg_ms else None
    plans = mm.muon_plan_query(shapes, ns_steps=ns_steps)[1]
    g_bytes = 2 if w.g_dtype == "bf16" else 4
    pair_bytes = sum(4 * p["m_pad"] * p["n_pad"] for p in plans if p["tile"] and ns_steps > 0)
    mom_bytes = w.n_params * (g_bytes + 8) + pair_bytes
    mom_gbps = mom_bytes / (stage_ms["momentum"] * 1e-3) / 1e9 if stage_ms["momentum"] else None
    rec = {
        "ms_per_step": round(ms_per_step, 4),
        "steps_per_s": round(1000.0 / ms_per_step, 3),
        "matrices_per_s": round(len(shapes) * 1000.0 / ms_per_step, 1),
        "steps": steps,
        "ns5_alg_tflop_per_step": round(ns_alg / 1e12, 4),
        "ns5_tflops": round(ns_tflops, 2) if ns_tflops else None,
        "ns5_frac_of_bf16_peak": round(ns_tflops / PEAK_BF16_TFLOPS, 4) if ns_tflops else None,
        "ns5_ms_per_step": round(ns_ms, 4),
        "step_tflops": round(ns_alg / (ms_per_step * 1e-3) / 1e12, 2),
        "bx_kernel_tflops": round(bx_tflops, 2) if bx_tflops else None,
        "bx_frac_of_bf16_peak": round(bx_tflops / PEAK_BF16_TFLOPS, 4) if bx_tflops else None,
        "momentum_gbps": round(mom_gbps, 1) if mom_gbps else None,
        "momentum_frac_of_hbm_peak": round(mom_gbps / PEAK_HBM_GBPS, 4) if mom_gbps else None,
        "momentum_frac_of_copy_ceiling": (round(mom_gbps / copy_ceiling, 4)
                                          if mom_gbps and copy_ceiling else None),
        "profiled_ms_per_step": round(prof_ms, 4),
        "profiling_overhead_ms": round(prof_ms - ms_per_step, 4),
        "stage_ms_per_step": {kk: round(v, 4) for kk, v in stage_ms.items() if v},
        "launches_per_step": {kk: v[1] / psteps for kk, v in prof.items() if v[1]},
    }
    if w.name in LATENCY_BOUND:
        rec["bound"] = "launch latency"
        rec["us_per_step"] = round(ms_per_step * 1e3, 2)
        rec["note"] = ("about 20 short launches of a few tiles each per step: the time is launch "
                       "latency, so the roofline fractions do not describe the kernels")
        # The same steps recorded once (muon_plan_create) and replayed as one
        # graph launch each: one plan per gradient buffer, each with its own
        # workspace (a plan's descriptor table lives there).
        gsets = grads if grads is not None else [[G for _, G, _, _ in mats]]
        recorded = [mm.muon_plan_create([(W, g[i], B, sc) for i, (W, _, B, sc) in enumerate(mats)],
                                     mu=w.mu, lr=w.lr, ns_steps=ns_steps) for g in gsets]
        for k in range(warmup):
            recorded[k % len(recorded)].step()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for k in range(steps):
            recorded[k % len(recorded)].step()
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / steps
        for pl in recorded:
            pl.close()
        rec["recorded_plan"] = {"ms_per_step": round(gms, 4), "us_per_step": round(gms * 1e3, 2),
                                "steps_per_s": round(1000.0 / gms, 2), "plans": len(recorded)}
        log(f"[bench] {w.name}: recorded plan replays, {gms * 1e3:.1f} us/step")
    if not headline:
        del mats, ws, grads
        torch.cuda.empty_cache()
        return rec

    # ---- the same step with per-matrix diagnostics (reported apart)
    if diag_steps > 0:
        dbuf = torch.zeros(len(shapes), 8, dtype=torch.int32, device=dev)

        def dstep():
            mm.muon_step_diag(mats, mu=w.mu, lr=w.lr, ns_steps=ns_steps, workspace=ws, diag=dbuf)

        dstep()
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(diag_steps):
            dstep()
        d1.record(stream)
        torch.cuda.synchronize()
        d_ms = d0.elapsed_time(d1) / diag_steps
        recs = mm.diag_records(dbuf, len(shapes))
        urms = [r["update_rms"] for r in recs]
        rec["diagnostics"] = {"steps": diag_steps, "ms_per_step": round(d_ms, 4),
                              "overhead_ms": round(d_ms - ms_per_step, 4),
                              "nonfinite_matrices": sum(1 for r in recs if r["nonfinite"]),
                              "update_rms_min": min(urms), "update_rms_max": max(urms)}
        log(f"[bench] with diagnostics: {d_ms:.3f} ms/step")
    bx_cfgs = sorted({(p["bx_tile_rows"], p["bx_tile_cols"]) for p in plans if p["tile"]})
    kname = "+".join(f"ns_gemm32_kernel<{BX_KERNEL_NAME[c]}, BX>" if c in BX_KERNEL_NAME
                     else f"ns_gemm_kernel<T{c[0]}, BX>" for c in bx_cfgs)
    rec["roofline"] = {
        "kernel": f"{kname} (X' = a X + P X)",
        "bound": "mfma",
        "achieved": round(bx_tflops, 2) if bx_tflops else None,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(bx_tflops / PEAK_BF16_TFLOPS, 4) if bx_tflops else None,
        "traffic": load_traffic(TRAFFIC_SOURCES, w.name),
        "avg_launch_ms": round(bx_avg_ms, 4) if bx_avg_ms else None,
        "launches_per_step": prof["bx"][1] / psteps,
        "alg_flops_per_launch": bx_flops_per_launch,
    }
    rec["ns5"] = {
        "alg_tflop_per_step": round(ns_alg / 1e12, 3),
        "tflops": round(ns_tflops, 2) if ns_tflops else None,
        "frac_of_bf16_peak": round(ns_tflops / PEAK_BF16_TFLOPS, 4) if ns_tflops else None,
        "effective_dense_tflops": round(dense_eq / (ns_ms * 1e-3) / 1e12, 2) if ns_ms else None,
        "ms_per_step": round(ns_ms, 4),
    }
    rec["config"] = {"workload": w.name, "matrices": len(shapes), "params": w.n_params,
                     "shapes": sorted({f"{r}x{c}" for r, c in shapes}), "ns_steps": ns_steps,
                     "mu": w.mu, "lr": w.lr, "g_dtype": w.g_dtype}
    del mats, ws, grads
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_xl_1p5b", choices=list(synth.ORDER),
                    help="the headline workload (value, roofline, cpu_baseline)")
    ap.add_argument("--only", action="store_true", help="time the headline workload alone")
    ap.add_argument("--ns-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--diag-steps", type=int, default=5,
                    help="after the timed steps, time this many steps with the per-matrix "
                         "diagnostics (muon_step_diag) and report their cost; 0 = skip")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain copy of this many MiB with the library's copy "
                         "kernel (counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--copy-calibration-mib; no GPU needed")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic, args.copy_calibration_mib * 2**20)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the Muon step of each matrix runs whole on one device).", file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_muon_step_amd as mm

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    mm.lib()
    dev = torch.device("cuda:0")

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib * 2**20
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        mm.muon_copy_probe(src, dst, 0)  # reads nb bytes, writes nb bytes
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {nb} bytes read, {nb} bytes written")
        del src, dst

    ceiling, ceiling_variant = copy_ceiling_gbps(dev)
    log(f"[bench] copy ceiling {ceiling:.0f} GB/s (variant {ceiling_variant})")
    names = [args.workload] if args.only else [n for n in synth.ORDER]
    records = {}
    for name in names:
        w = synth.WORKLOADS[name]
        head = name == args.workload
        steps = args.steps if head else DEFAULT_STEPS[name]
        records[name] = bench_workload(w, steps, args.warmup, args.ns_steps, dev, head,
                                       diag_steps=args.diag_steps if head else 0, copy_ceiling=ceiling)
    h = records[args.workload]
    w = synth.WORKLOADS[args.workload]
    out = {
        "metric": METRIC,
        "value": h["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (low-rank plus noise gradients drawn on the GPU, random-init fp32 weights)",
        "config": h.pop("config"),
        "roofline": h.pop("roofline"),
        "ns5": h.pop("ns5"),
        "matrices_per_s": h["matrices_per_s"],
        "stage_ms_per_step": h["stage_ms_per_step"],
        "launches_per_step": h["launches_per_step"],
        "profiled_ms_per_step": h["profiled_ms_per_step"],
        "elementwise": {
            "momentum_gbps": h["momentum_gbps"],
            "copy_ceiling_gbps": round(ceiling, 1),
            "copy_ceiling_kernel": f"muon_copy_probe variant {ceiling_variant}",
            "momentum_frac_of_hbm_peak": h["momentum_frac_of_hbm_peak"],
            "momentum_frac_of_copy_ceiling": h["momentum_frac_of_copy_ceiling"],
        },
        "hbm_peak_gbps": PEAK_HBM_GBPS,
        "diagnostics": h.pop("diagnostics", None),
        "workloads": records,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
