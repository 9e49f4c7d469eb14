#!/usr/bin/env python
"""DyRA layer-forward benchmark on one MI355X.  Prints ONE JSON line.

A step is one full DyRA forward (stage-1 pass, token reductions, r x r solve,
right-factor GEMM, fused output GEMM) over one batch of synthetic input of the
ViT-L/16 (DINOv3-like, 1029 tokens per image) MLP fc1 shape: B = 32 images,
X (32*1029) x 1024 -> Y (32*1029) x 4096, low-rank static rank 256, residual
rank 64, bf16 storage with fp32 accumulation.  Inputs and the prepared plan
are resident in HBM before the timed region starts.

Extra legs (excluded from `value`): per-stage HIP-event timing of the same
launches (the roofline of the dominant kernel), the dense X W comparators
(the library's own MFMA GEMM and torch.matmul / hipBLASLt), and the float64
oracle timed on the host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
WORKLOAD_TEXT = {
    "tiny_fp32": "tiny fp32 layer",
    "vitb_fc1": "ViT-B/16 MLP fc1",
    "vitl_fc1": "ViT-L/16 MLP fc1",
    "vitl_fc2": "ViT-L/16 MLP fc2",
    "monarch": "Monarch 32 x (32 x 32) layer at the ViT-L token count",
    "lm_blast": "LM prefill QKV-shaped layer, BLAST 16 x 16 grid, rank 128",
    "lm_blast_diag": "LM prefill QKV-shaped layer, BLAST 16 x 16 grid, rank 128, diagonal couplings",
}
STAGES = ["stage1_X_UP", "token_reductions_M_G", "solve_apply", "right_factor_R", "fused_output_Y"]


def stage_work(w):
    """Algorithmic flops and HBM bytes of each event-timed stage for one
    launch (one batch of B segments); bf16 = 2 bytes, fp32 = 4 bytes."""
    from input_adaptive_rank_amd import synth
    e = 2 if w.dtype == 1 else 4
    n, c1, c2, r, B = w.n, w.c1, w.c2, w.r, w.B
    # shared by every structure: M_b, G_b; the r x r solve and M' = Ginv M;
    # R^T = W_res^T M'^T for all segments at once
    s3 = (2 * n * r * c1 + 2 * n * r * r, e * (n * c1 + r * n) + 4 * (B * r * c1 + B * r * r))
    s4 = (B * (2 * r ** 3 + 2 * r * r * c1), 4 * (2 * B * r * r + B * r * c1) + e * B * r * c1)
    s5 = (2 * c2 * B * r * c1, e * (c2 * c1 + B * r * c1 + c2 * B * r))
    if w.kind == synth.KIND_MONARCH:
        m = w.mblk   # c = m^2: stage 1 and stage 2 are m block products of m x m
        s1 = (2 * n * c1 * m + 2 * n * c1 * r, e * (n * c1 + c1 * m + c1 * r + n * (c1 + r) + r * n))
        s6 = (2 * n * c2 * m + 2 * n * r * c2, e * (n * (c1 + r) + c2 * m + c2 * B * r + c2 + n * c2))
    elif w.kind in (synth.KIND_BLAST, synth.KIND_BLAST_DIAG):
        nr = w.nb * w.rb  # Z = X blockdiag(U_i): n x (nb rb); coupling W' = Z S
        s1 = (2 * n * c1 * w.rb + 2 * n * c1 * r, e * (n * c1 + c1 * w.rb + c1 * r + n * (nr + r) + r * n))
        if w.kind == synth.KIND_BLAST:     # full rb x rb couplings: one (nb rb)^2 GEMM
            cpl = (2 * n * nr * nr, e * (2 * n * nr + nr * nr))
        else:                              # diagonal couplings: nb^2 rb weights
            cpl = (2 * n * w.nb * nr, e * (2 * n * nr + w.nb * nr))
        s5 = (s5[0] + cpl[0], s5[1] + cpl[1])   # the coupling GEMM runs in the same event interval
        s6 = (2 * n * w.rb * c2 + 2 * n * r * c2, e * (n * nr + n * r + c2 * w.rb + c2 * B * r + c2 + n * c2))
    else:
        N = w.k + r
        s1 = (2 * n * c1 * N, e * (n * c1 + N * c1 + n * N + r * n))
        s6 = (2 * n * N * c2, e * (n * N + c2 * w.k + c2 * B * r + c2 + n * c2))
    return {"stage1_X_UP": s1, "token_reductions_M_G": s3, "solve_apply": s4, "right_factor_R": s5,
            "fused_output_Y": s6}


def STRUCT_TEXT(w):
    return {0: f"low-rank k={w.k}", 1: f"Monarch {w.mblk} x ({w.mblk} x {w.mblk})",
            2: f"BLAST {w.nb} x {w.nb} grid, rb={w.rb}",
            3: f"BLAST {w.nb} x {w.nb} grid, rb={w.rb}, diagonal couplings"}[w.kind]


OUTPUT_KERNEL = {0: "s6_lowrank_kernel (fused T V + L R_b + bias)",
                 "0bf16": "s6_lowrank_ws_kernel (persistent, wave-specialised T V + L R_b + bias)",
                 1: "s6_monarch_fused_kernel (stage 1 recomputed from X, V_j B2_j + L R_b + bias)",
                 2: "s6_lowrank_ws_kernel (persistent: W'_j V_j^T + L R_b + bias)",
                 3: "s6_lowrank_ws_kernel (persistent: W'_j V_j^T + L R_b + bias)"}


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "input_adaptive_rank_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")) and f not in ("host_linalg.h",):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def profile_record(workload, kernel_hash):
    """The machine-readable block of the committed rocprofv3 summary for this
    workload (profiles/forward_<workload>.md), or None when it is absent or
    was taken on other kernel code (its kernel source hash differs)."""
    path = os.path.join(ROOT, "profiles", f"forward_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    return d if d.get("kernel_source_hash") == kernel_hash else None


def cpu_baseline(w, budget_s=12.0, t=1.0):
    """The float64 oracle forward on the host cores, on the same workload."""
    from input_adaptive_rank_amd import synth
    from oracle import dyra_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:   # noqa: BLE001
        threads = os.cpu_count()
    inp = synth.make_inputs(w)
    prep = O.prepare(inp.W, w.kind, w.r, k=w.k, mblk=w.mblk, nb=w.nb, rb=w.rb)
    t0 = time.perf_counter()
    runs = 0
    while True:
        Y = O.forward(inp.X, prep, inp.bias, w.B, w.s, eps=1e-6, t=t)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 3:
            break
    return {"value": round(w.n * runs / el, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full {w.name} batch ({w.B} x {w.s} tokens), float64 numpy oracle forward (ALS t = {t}), "
                      f"{runs} run(s) in {el:.2f} s (prepare excluded)"}, Y


def parity_vs_oracle(w, Yg, Y_or):
    """End-to-end error of the timed output against the oracle's forward
    (which ran its own float64 prepare): whole output and worst segment."""
    d = Yg - Y_or
    seg = max(float(np.linalg.norm(d[b * w.s:(b + 1) * w.s]) / np.linalg.norm(Y_or[b * w.s:(b + 1) * w.s]))
              for b in range(w.B))
    return {"rel_fro": float(np.linalg.norm(d) / np.linalg.norm(Y_or)), "seg_rel_max": seg,
            "reference": "float64 oracle forward with its own float64 prepare (end to end)",
            "bar": 2e-2 if w.dtype == 1 else 1e-4}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="vitl_fc1")
    ap.add_argument("--solver", choices=["auto", "chol", "ns"], default=None,
                    help="r x r solver (default: the workload's own choice)")
    ap.add_argument("--als-half-steps", type=int, default=2,
                    help="2 t ALS half-steps (2: t = 1, the default; 3: t = 1.5; 4: t = 2; low-rank bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time only eager forwards (no HIP graph replay)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "the DyRA forward would shard by segments, with no communication between GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from input_adaptive_rank_amd import dyra as D
    from input_adaptive_rank_amd import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    t0 = time.perf_counter()
    factors = D.prepare(inp.W, D.spec_of(w))
    prep_s = time.perf_counter() - t0
    solver = args.solver or w.solver
    layer = D.DyraLayer(D.spec_of(w), factors, w.dtype, bias=inp.bias, device=dev, solver=D.SOLVERS[solver],
                        half_steps=args.als_half_steps)
    als = args.als_half_steps != 2
    tdt = D.torch_dtype(w.dtype)
    # 4 input/output buffer sets so X is not cache-resident from the previous step
    NB = 4
    X0 = D.to_device(inp.X, w.dtype, dev)
    Xs = [X0] + [X0.clone() for _ in range(NB - 1)]
    Ys = [torch.empty((w.n, w.c2), dtype=tdt, device=dev) for _ in range(NB)]
    layer.workspace(w.B, w.s)
    stream = torch.cuda.current_stream()

    for i in range(args.warmup):
        layer.forward(Xs[i % NB], w.B, w.s, out=Ys[i % NB])
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for row in ev:           # create the HIP events
        for e in row:
            e.record(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region 1, the headline: K plain forwards (what a caller runs)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        layer.forward(Xs[i % NB], w.B, w.s, out=Ys[i % NB])
    end.record(stream)
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / K
    ms = ms_eager
    # timed region 1b: the same K forwards replayed from HIP graphs (one per
    # buffer set), which removes the host launch gaps between the stages.
    # Every graph's output is first checked bit for bit against an eager
    # forward of the same inputs, with eager work between the replays; on any
    # mismatch or capture failure the eager timing stays the headline.
    launch, graph_note = "eager", None
    if not args.no_graph:
        try:
            graphs = []
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for i in range(NB):
                    layer.forward(Xs[i], w.B, w.s, out=Ys[i])
            stream.wait_stream(side)
            torch.cuda.synchronize()
            for i in range(NB):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    layer.forward(Xs[i], w.B, w.s, out=Ys[i])
                graphs.append(g)
            torch.cuda.synchronize()
            ok = True
            for rep in range(3):
                for i in range(NB):
                    ref = layer.forward(Xs[i], w.B, w.s)
                    torch.cuda.synchronize()
                    Ys[i].fill_(0)
                    graphs[i].replay()
                    torch.cuda.synchronize()
                    ok = ok and bool(torch.equal(Ys[i], ref))
            if ok:
                for i in range(args.warmup):
                    graphs[i % NB].replay()
                torch.cuda.synchronize()
                start.record(stream)
                for i in range(K):
                    graphs[i % NB].replay()
                end.record(stream)
                torch.cuda.synchronize()
                ms = start.elapsed_time(end) / K
                launch = "hip_graph"
            else:
                graph_note = "graph replay differed from the eager forward; eager timing reported"
        except Exception as exc:   # capture unsupported: keep the eager number
            graph_note = f"graph capture failed ({type(exc).__name__}); eager timing reported"
    # timed region 2: the same K steps with HIP events recorded between the
    # stages on the launch stream (per-stage times and the roofline kernel time)
    # -- for the t = 1 forward, whose stage boundaries the events mark
    ms_events, stage_ms, step_pct = None, None, None
    if not als:
        start.record(stream)
        for i in range(K):
            layer.forward_events(Xs[i % NB], w.B, w.s, Ys[i % NB], ev[i], stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms_events = start.elapsed_time(end) / K
        stage_ms = {STAGES[j]: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]))
                    for j in range(5)}
        # per-step spread of the same pass (first to last stage event)
        steps = np.array([ev[i][0].elapsed_time(ev[i][5]) for i in range(K)])
        step_pct = {f"p{q}": round(float(np.percentile(steps, q)), 5) for q in (10, 50, 90)}
    status = layer.status(w.B, w.s)

    work = stage_work(w)
    total_flops = sum(v[0] for v in work.values())
    khash = kernel_source_hash()
    stages, roof = None, None
    if not als:
        stages = {}
        for name, (fl, by) in work.items():
            t = stage_ms[name] * 1e-3
            stages[name] = {"ms": round(stage_ms[name], 5), "TFLOP/s": round(fl / t / 1e12, 1),
                            "GB/s": round(by / t / 1e9, 1), "gflop": round(fl / 1e9, 3), "mb": round(by / 1e6, 2)}
        # roofline of the dominant kernel: the fused output GEMM (Y = [T|L][V;R_b] + bias)
        fl, by = work["fused_output_Y"]
        t6 = stage_ms["fused_output_Y"] * 1e-3
        t_mfma, t_hbm = fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9)
        rec = profile_record(w.name, khash)
        out6 = (rec or {}).get("fused_output") or {}
        hbm = t_hbm >= t_mfma
        if hbm:
            roof = {"bound": "hbm", "achieved": round(by / t6 / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": round(fl / t6 / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s"}
        # headline frac: event-timed in this run; beside it the same ratio
        # from the committed rocprofv3 kernel-trace average of this kernel code
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["frac_source"] = "HIP events around the kernel's launch in this run (average over the timed steps)"
        if out6.get("avg_us"):
            t6r = out6["avg_us"] * 1e-6
            roof["frac_rocprof"] = round((by / t6r / 1e9 / PEAK_HBM_GBS) if hbm else
                                         (fl / t6r / 1e12 / PEAK_BF16_TFLOPS), 4)
            roof["rocprof_avg_us"] = out6["avg_us"]
        roof["traffic"] = out6.get("traffic_bytes")
        roof["kernel"] = OUTPUT_KERNEL["0bf16" if (w.kind == 0 and w.dtype == synth.DT_BF16) else w.kind]
        roof["mfma_frac"] = round(fl / t6 / 1e12 / PEAK_BF16_TFLOPS, 4)
        if out6.get("mfma_busy_frac") is not None:
            roof["mfma_busy_frac_counters"] = out6["mfma_busy_frac"]

    # dense comparators on the same shape: library MFMA GEMM and torch.matmul (hipBLASLt)
    dense = None
    if not args.no_dense:
        Wt = D.to_device(np.ascontiguousarray(inp.W.T), w.dtype, dev)
        bias_d = layer.bias
        Yd = torch.empty((w.n, w.c2), dtype=tdt, device=dev)

        def timeit(fn, iters):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(iters):
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / iters

        it = max(10, K // 2)
        ms_ref = timeit(lambda i: D.dense_ref(Xs[i % NB], Wt, bias_d, Ys[i % NB], w.dtype), it)
        if bias_d is not None:
            ms_torch = timeit(lambda i: torch.addmm(bias_d, Xs[i % NB], Wt.t(), out=Yd), it)
        else:
            ms_torch = timeit(lambda i: torch.matmul(Xs[i % NB], Wt.t(), out=Yd), it)
        best = min(ms_ref, ms_torch)
        dense = {"dyra_dense_ref_ms": round(ms_ref, 5), "torch_matmul_ms": round(ms_torch, 5),
                 "dense_gflop": round(2 * w.n * w.c1 * w.c2 / 1e9, 1),
                 "speedup_vs_dense": round(best / ms, 3)}

    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    parity = None
    if args.no_cpu_baseline:
        cpu = None
    else:
        cpu, Y_or = cpu_baseline(w, t=args.als_half_steps / 2)
        Yg = layer.forward(Xs[0], w.B, w.s)
        torch.cuda.synchronize()
        parity = parity_vs_oracle(w, Yg.float().cpu().numpy().astype(np.float64), Y_or)

    out = {
        "metric": "DyRA layer tokens/s + % bf16 MFMA peak at ViT-L shape; speedup vs dense XW",
        "value": round(w.n / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_with_stage_events": None if ms_events is None else round(ms_events, 5),
        "step_ms_with_stage_events": step_pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == synth.DT_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {WORKLOAD_TEXT.get(w.name, 'DyRA layer')}, B={w.B} x {w.s} tokens, "
                               f"{w.c1}->{w.c2}, {STRUCT_TEXT(w)}, r={w.r}, "
                               f"{'bf16' if w.dtype == synth.DT_BF16 else 'fp32'}, fp32 accumulate",
                   "global_batch": w.B, "seq_len": w.s, "tokens": w.n, "solver": solver,
                   "als_t": args.als_half_steps / 2, "launch": launch},
        "tflops": None if als else round(total_flops / (ms * 1e-3) / 1e12, 1),
        "pct_bf16_peak": None if als else round(100 * total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "dense": dense,
        "speedup_vs_dense": dense["speedup_vs_dense"] if dense else None,
        "stages": stages,
        "solver_status_ok": bool(np.all(status == 0)),
        "kernel_source_hash": khash,
        "prepare_s": round(prep_s, 2),
        "gpu": torch.cuda.get_device_name(0),
    }
    if graph_note:
        out["graph_note"] = graph_note
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
