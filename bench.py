#!/usr/bin/env python3
"""Benchmark of the MoE expert-FFN layer on one MI355X.

One step = one full forward of the layer (route -> gathered up_proj GEMM with
SwiGLU -> down_proj GEMM -> combine) on a seeded synthetic batch that is
already resident in HBM; for the forward+backward workload also the backward.
The forward runs as the library does by default: route, the two grouped
GEMMs and the combine as separate launches, or on 64-row tiles (the
weight-streaming decode shape) route, the two GEMMs as one pipelined launch
with tile-granular release, and the combine.  The step is timed eagerly (with
per-stage HIP events) and as a HIP graph replay of the same calls (every
kernel runs every step; only the host-side launch work is gone); the headline
is the replay when its output equals the eager output bit for bit.  The other
mode (pipelined or two launches) is timed eagerly after it and reported as
"twin".  Prints ONE JSON line.

Default workload: prefill, bf16 with fp32 accumulation, T=4096 tokens,
H=2048, I=1408, E=64 experts, K=6, uniform routing.  Other workloads:
--workload {tiny_f32,prefill_bf16,skewed_bf16,decode_bf16,fwdbwd_bf16}.

Besides tokens/s the line carries
* "roofline": the dominant kernel (the up_proj GEMM with its SwiGLU epilogue,
  or the pipelined launch where it is the default; against HBM bandwidth for
  the HBM-bound decode shape), its algorithmic work per launch divided by its
  average launch time, where the launch times come from HIP events that the library
  records around that kernel on the call's stream during the timed steps;
* "stage_roofline": each bulk forward stage (GEMM1, GEMM2, combine) against
  both bounds, from its algorithmic bytes and flops per launch;
* "cpu_baseline": the CPU oracle on the host's cores over a bounded sample of
  the same workload (its first tokens), unless --no-cpu-baseline;
* with the default workload, "decode": the same record (ms/step, the layer's
  fraction of peak HBM bandwidth, roofline of each kernel, cpu_baseline) for
  the weight-streaming decode shape (T=128, H=7168, I=2048, E=32, K=8),
  measured in the same process after the prefill record (--no-decode skips
  it).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-FFN layer tokens/s + % peak MFMA (prefill) / % peak HBM BW (decode)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one by one after evicting the caches (512 MiB written "
                         "between steps, outside the timed region); 0 to skip")
    ap.add_argument("--no-decode", action="store_true",
                    help="with the default prefill workload, skip the decode record that "
                         "otherwise follows it in the same line")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one elementwise copy of this many MiB (for scaling HBM "
                         "byte counters against a kernel of known traffic)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the layer is measured on exactly one GPU (one GPU's share of the "
              "experts); multi-GPU runs are not supported (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401

    import mixture_experts_ffn_amd as m

    m.load_library()
    out = measure(args.workload, args, primary=True)
    # The metric's HBM half: the weight-streaming decode shape, measured in the
    # same process after the default (prefill) workload
    if args.workload == "prefill_bf16" and not args.no_decode:
        dec = measure("decode_bf16", args, primary=False)
        out["decode"] = {k: dec[k] for k in ("value", "unit", "ms_per_step", "config", "layer",
                                              "launch", "eager", "graph_replay",
                                              "twin", "roofline", "stage_roofline",
                                              "cpu_baseline", "hbm_reference")
                         if k in dec}
    print(json.dumps(out), flush=True)


def measure(workload_name, args, primary):
    """Time one workload; returns the bench record (metric, value, roofline, ...)."""
    import torch

    import mixture_experts_ffn_amd as m
    from synth import make_inputs, workload

    w = workload(workload_name)
    inp = make_inputs(w, with_dy=w.backward)
    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    d = {k: to_dev(v) for k, v in inp.items()}
    prob = m.make_problem(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"])
    prob.Is = w.Is
    ws_bytes, _ = m.fwd_workspace_size(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tile_rows, kernel_family = m.fwd_plan(prob)

    bws = None
    if w.backward:
        bws = torch.empty(max(m.bwd_workspace_size(prob), 1), dtype=torch.uint8, device=dev)

    sh = ({"shared_up_proj_weight": d["shared_up"], "shared_down_proj_weight": d["shared_down"]}
          if w.Is else {})
    def step(ev=None, bev=None, pipelined=None):
        if not w.backward:
            return m.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                 d["down_proj"], ws=ws, stage_events=ev, pipelined=pipelined,
                                 **sh)
        y, saved = m.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                 d["down_proj"], ws=ws, stage_events=ev, save_for_backward=True,
                                 pipelined=pipelined, **sh)
        m.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                      d["down_proj"], saved, ws=bws, stage_events=bev, **sh)
        return y

    def stats(ms):
        ms = np.asarray(ms, np.float64)
        return {"median": float(np.median(ms)), "min": float(ms.min()),
                "p90": float(np.percentile(ms, 90)), "n": int(ms.size)}

    def timed(pipelined):
        """warmup, then the timed steps; per-stage mean ms from the library's events
        and per-step times from events around each step (same stream)"""
        for _ in range(args.warmup):
            step(pipelined=pipelined)
        torch.cuda.synchronize()
        pool = m.EventPool(args.steps)
        bpool = m.EventPool(args.steps, n_stages=len(m.BWD_STAGES)) if w.backward else None
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        marks[0].record()
        for i in range(args.steps):
            y = step(pool.sets[i], bpool.sets[i] if bpool else None, pipelined=pipelined)
            marks[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        per_step = stats([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
        stages = {}
        for s, name in enumerate(m.STAGES):
            try:  # stages a path does not run are never recorded
                stages[name] = float(np.mean([pool.elapsed_ms(i, s) for i in range(args.steps)]))
            except m.MoEFFNError:
                pass
        pool.close()
        if bpool:
            stages.update({"bwd_" + name: float(np.mean([bpool.elapsed_ms(i, s)
                                                         for i in range(args.steps)]))
                           for s, name in enumerate(m.BWD_STAGES)})
            bpool.close()
        return y, elapsed, stages, per_step

    def cold(n):
        """steps timed one by one, each after writing 512 MiB (more than the 256 MB
        last-level cache) outside the timed region"""
        scratch = torch.empty(512 * (1 << 20) // 4, dtype=torch.float32, device=dev)
        ms = []
        for _ in range(n):
            scratch.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        del scratch
        return stats(ms)

    # the first call of the process (code-object load, first-touch of the
    # workspace), timed on its own
    fa, fb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    fa.record()
    step()
    fb.record()
    torch.cuda.synchronize()
    first_call_ms = fa.elapsed_time(fb)

    # the library's default forward is the measured one (for this workload the
    # one pipelined launch or the two GEMM launches, whichever it picks); the
    # other mode, its twin, is timed after it
    def graphed():
        """The default step captured once into a HIP graph and replayed: the same
        kernels every step, without per-launch host work.  Returns the replayed
        output (checked against the eager step) and the time of the replays."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            yg = step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        return yg, time.perf_counter() - t0

    default_pipelined = m.fwd_plan(prob)[1] == "pipelined"
    y, elapsed, stage_ms, step_stats = timed(pipelined=None)
    twin_pipelined = not default_pipelined
    _, twin_elapsed, twin_stage_ms, _ = timed(pipelined=twin_pipelined)
    cold_stats = cold(args.cold_steps) if args.cold_steps > 0 else None
    y_graph, graph_elapsed = graphed()
    graph_ok = bool(torch.equal(y_graph, y))

    eager_ms = elapsed / args.steps * 1e3
    # the headline: graph replay of the default step when it reproduces the
    # eager output bit for bit, else the eager step
    step_s = graph_elapsed if graph_ok else elapsed
    ms_per_step = step_s / args.steps * 1e3
    tokens_per_s = w.T * args.steps / step_s
    counts = np.bincount(inp["topk_ids"].ravel(), minlength=w.E)
    live = counts > 0
    es = 2 if w.dtype == "bf16" else 4
    layer_flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)
    layer_bytes = ((live.sum() * w.I + w.Is) * 3 * w.H * es + 2 * w.T * w.H * es
                   + w.T * w.K * 8)
    nl = live.sum() * w.I + w.Is
    TKp = w.T * (w.K + w.Is // w.I)
    g1_bytes = nl * w.H * 2 * es + w.T * w.H * es + TKp * w.I * es
    g2_bytes = nl * w.H * es + TKp * w.I * es + TKp * w.H * es
    cb_bytes = TKp * w.H * es + w.T * w.H * es + w.T * w.K * 8
    if "pipeline" in stage_ms:
        # dominant kernel: the pipelined launch (both grouped GEMMs; the
        # combine is a launch of its own)
        k_flops = w.fwd_flops()
        k_bytes = g1_bytes + g2_bytes
        k_ms = stage_ms["pipeline"]
        kernel = (f"moe::fast::moe_fwd_bf16<{tile_rows}, FAST_PIPE> "
                  "(GEMM1+SwiGLU, GEMM2 in one launch)")
    else:
        # dominant kernel: the gathered up_proj GEMM with the SwiGLU epilogue
        # (one launch covers the routed experts and the shared expert's chunks)
        k_flops = 4.0 * w.T * w.H * (w.K * w.I + w.Is)
        k_bytes = g1_bytes
        k_ms = stage_ms["gemm1"]
        mode = "FAST_G1H" if w.backward else "FAST_G1"  # the training forward also saves h
        g1_tiles = (f"moe::fast::moe_fwd_bf16<{tile_rows}, {mode}> "
                    "(gathered up_proj GEMM + SwiGLU)")
        kernel = {"tiles": g1_tiles,
                  "tiles_big_gemm2": g1_tiles,
                  "big_tiles": f"moe::big::moe_fwd_bf16_big<{mode}, false> "
                               "(gathered up_proj GEMM + SwiGLU, 256 x 256 tiles)",
                  }.get(kernel_family, f"up_proj GEMM + SwiGLU ({kernel_family} kernel)")
    if w.name.startswith("decode"):
        roof = {"bound": "hbm", "achieved": k_bytes / (k_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": k_flops / (k_ms * 1e-3) / 1e12, "peak": peak,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    dom_role = "pipeline" if "pipeline" in stage_ms else "gemm1"
    dom_src = "gemm_big.hip" if kernel_family == "big_tiles" else "gemm_mfma.hip"
    roof["traffic"] = measured_traffic(w.name, dom_role, dom_src, tile_rows)
    # the clock the kernel ran at under the power cap, and how busy its matrix
    # cores were (what separates the clock from the kernel's own efficiency)
    roof["clock_ghz"], roof["mfma_busy"] = measured_clock(w.name, dom_role, dom_src, tile_rows)
    roof["kernel"] = kernel
    roof["avg_launch_ms"] = k_ms
    # every stage of the bulk forward against its own bound: algorithmic bytes
    # (weights of live experts, activations in and out) or flops per launch
    stage_roof = {}
    g1_flops = 4.0 * w.T * w.H * (w.K * w.I + w.Is)
    for name, nbytes, nflops in (("gemm1", g1_bytes, g1_flops),
                                 ("gemm2", g2_bytes, g1_flops / 2),
                                 ("pipeline", g1_bytes + g2_bytes, 1.5 * g1_flops),
                                 ("combine", cb_bytes, 0.0)):
        if name in stage_ms:
            t = stage_ms[name] * 1e-3
            stage_roof[name] = {"ms": stage_ms[name], "hbm_gbs": nbytes / t / 1e9,
                                "hbm_frac": nbytes / t / 1e9 / PEAK_HBM_GBS,
                                "tflops": nflops / t / 1e12,
                                "mfma_frac": nflops / t / 1e12 / (
                                    PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS)}

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy PCG64; random-init weights)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "K": w.K,
                   "routing": w.routing, "accumulate": "f32",
                   "step": "forward + backward" if w.backward else "forward"},
        "layer": {"tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
                  "frac_mfma": layer_flops / (ms_per_step * 1e-3) / 1e12 /
                  (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS),
                  "hbm_gbs_alg": layer_bytes / (ms_per_step * 1e-3) / 1e9,
                  "stage_ms": stage_ms},
        "launch": "hip_graph_replay" if graph_ok else "eager",
        "eager": {"ms_per_step": eager_ms, "tokens_per_s": w.T * args.steps / elapsed,
                  "step_ms": step_stats, "first_call_ms": first_call_ms,
                  "cold_step_ms": cold_stats},
        "graph_replay": {"ms_per_step": graph_elapsed / args.steps * 1e3,
                         "tokens_per_s": w.T * args.steps / graph_elapsed,
                         "output_equals_eager": graph_ok},
        "twin": {"mode": "pipelined" if twin_pipelined else "bulk",
                 "plan": m.fwd_plan(prob, m.PIPELINE if twin_pipelined else m.BULK),
                 "ms_per_step": twin_elapsed / args.steps * 1e3,
                 "tokens_per_s": w.T * args.steps / twin_elapsed,
                 "stage_ms": twin_stage_ms},
        "roofline": roof,
        "stage_roofline": stage_roof,
        "cpu_baseline": None,
    }
    if w.name.startswith("decode"):
        # the HBM half of the metric: the whole layer's algorithmic bytes per step
        out["layer"]["hbm_frac_alg"] = out["layer"]["hbm_gbs_alg"] / PEAK_HBM_GBS

    if w.dtype == "bf16" and not w.name.startswith("decode"):
        out["dense_reference"] = dense_reference(w, dev)
    if w.name.startswith("decode"):
        out["hbm_reference"] = hbm_reference(dev)

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        torch.add(src, 0.0, out=dst)  # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        out["copy_calibration"] = {"bytes_read": n * 4, "bytes_written": n * 4}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, y, args.cpu_seconds)
    return out


def dense_reference(w, dev, reps=20):
    """Context only: torch.matmul (the vendor BLAS) on the dense bf16 GEMMs of the
    same total size, [R, H] x [H, 2I] and [R, I] x [I, H] with R = T*K (+ T*Is/I
    with a shared expert), as an achievable
    rate for comparison with the grouped kernels."""
    import torch

    out = {}
    rows = w.T * w.K + w.T * (w.Is // w.I)  # the shared expert's chunks add T rows each
    for name, (M, Kd, N) in {"gemm1": (rows, w.H, 2 * w.I),
                             "gemm2": (rows, w.I, w.H)}.items():
        a = torch.randn(M, Kd, device=dev, dtype=torch.bfloat16)
        b = torch.randn(Kd, N, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / reps * 1e3
        out[name] = {"shape": [M, Kd, N], "ms": ms,
                     "tflops": 2.0 * M * Kd * N / (ms * 1e-3) / 1e12}
        del a, b
    return out


def hbm_reference(dev, mib=2048, reps=10):
    """Context only: a large device-to-device copy (torch's copy kernel), as an
    achievable HBM rate for comparison with the weight-streaming decode GEMMs."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.empty(n, device=dev, dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    del src, dst
    return {"bytes_moved": 2 * n * 4, "ms": ms, "gbs": 2 * n * 4 / (ms * 1e-3) / 1e9}


def profile_entry(table_name, workload_name, kernel, source, tile_rows):
    """The values a committed rocprofv3 summary table (profiles/<table_name>)
    holds for this workload and kernel role, or None when the kernel source
    has changed since the counters were taken, the line was taken with
    another tile height (one source holds the kernels of several heights) or
    the table has no such line.
    Lines: workload role source:sha1[:12] tile_rows=N name=value ..."""
    import hashlib

    src = os.path.join(ROOT, "mixture_experts_ffn_amd", "csrc", source)
    table = os.path.join(ROOT, "profiles", table_name)
    if not (os.path.exists(src) and os.path.exists(table)):
        return None
    sha = hashlib.sha1(open(src, "rb").read()).hexdigest()[:12]
    for line in open(table):
        parts = line.split()
        if (len(parts) >= 4 and parts[0] == workload_name and parts[1] == kernel
                and parts[2] == f"{source}:{sha}"):
            e = {k: float(v) for k, v in (p.split("=") for p in parts[3:])}
            if e.get("tile_rows") == tile_rows:
                return e
    return None


def measured_traffic(workload_name, kernel, source, tile_rows):
    """HBM bytes per launch of the dominant kernel from the committed PMC summary
    (profiles/traffic.txt: FETCH_SIZE and WRITE_SIZE, scaled against a copy of
    known size), or None when stale or absent."""
    e = profile_entry("traffic.txt", workload_name, kernel, source, tile_rows)
    return None if e is None else e["fetch_bytes"] + e["write_bytes"]


def measured_clock(workload_name, kernel, source, tile_rows):
    """Shader clock (GHz) and matrix-core busy fraction of the dominant kernel
    from the committed PMC summary (profiles/clock.txt: GRBM_GUI_ACTIVE and
    SQ_VALU_MFMA_BUSY_CYCLES over the dispatch), or (None, None) when stale or
    absent."""
    e = profile_entry("clock.txt", workload_name, kernel, source, tile_rows)
    return (None, None) if e is None else (e["clock_ghz"], e["mfma_busy"])


def cpu_baseline(w, inp, y_gpu, target_s):
    """The CPU oracle on the first n tokens of the same batch (n sized for ~target_s)."""
    import oracle

    def run(n):
        t0 = time.perf_counter()
        if w.Is:
            yo = oracle.forward_shared(inp["x"][:n], inp["topk_ids"][:n],
                                       inp["topk_weights"][:n], inp["up_proj"], inp["down_proj"],
                                       inp["shared_up"], inp["shared_down"])
        else:
            yo = oracle.forward(inp["x"][:n], inp["topk_ids"][:n], inp["topk_weights"][:n],
                                inp["up_proj"], inp["down_proj"])
        return yo, time.perf_counter() - t0

    n = min(w.T, 8)
    _, dt = run(n)
    while dt < 0.5 and n < w.T:
        n = min(w.T, n * 4)
        _, dt = run(n)
    n = int(min(w.T, max(1, n * target_s / max(dt, 1e-6))))
    yo, dt = run(n)
    got = y_gpu[:n].float().cpu().numpy().astype(np.float64)
    err = float(np.abs(got - yo).max() / max(np.abs(yo).max(), 1e-300))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": model,
            "sample": f"first {n} of {w.T} tokens of the same batch (all {w.E} experts' weights), "
                      f"{dt:.1f} s, fp64 accumulation",
            "max_rel_err_gpu_vs_oracle_on_sample": err}


if __name__ == "__main__":
    main()
