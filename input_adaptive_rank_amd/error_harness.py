"""Approximation-error harness for the DyRA layer on synthetic layers.

Two measurements from the paperlayer.ai summary of the DyRA paper, both taken
on outputs the GPU library computes (dyra_forward_als, dyra_dense_ref):

E.3 ("Convergence of ALS Residual Approximation"): for t = 1, 1.5, 2 ALS
    iterations, the relative Frobenius error of the correction L(t) R(t)
    against the residual product X W_res, beside the optimal rank-r error
    from an SVD of X W_res (Eckart-Young), per segment then averaged.
E.4 ("FLOPs-Matched Output Approximation Error", Figure 3): the normalised
    output error ||X W + b - Y||_F / ||X W + b||_F of DyRA (t = 1) against a
    static low-rank layer whose rank k' is raised until its FLOPs reach
    DyRA's total FLOPs, correction overhead included.

Here W_res is the residual the device actually corrects, W - W_hat with W_hat
as stored (bf16 factors), so ||X W + b - Y|| = ||X W_res - L R|| up to the
rounding of Y; the exact products are float64 numpy on the host.  Usage:

    python -m input_adaptive_rank_amd.error_harness --workloads vitb_fc1,vitl_fc1,vitl_fc2 --segments 4

prints one JSON line per workload.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

from . import dyra as D
from . import synth


def dyra_flops_per_segment(s: int, c1: int, c2: int, k: int, r: int) -> float:
    """Algorithmic flops of one low-rank DyRA segment (multiply-add = 2):
    [T | L] = X [U | P], G = L^T L, M = L^T X, the r x r Cholesky solve and
    (G + lambda I)^-1 M, R = M' W_res, and Y = T V + L R."""
    return (2 * s * c1 * (k + r) + 2 * s * r * r + 2 * s * r * c1 + 2 * r * c1 * c2
            + (r ** 3 / 3 + 2 * r * r * min(c1, c2)) + 2 * s * (k + r) * c2)


def static_flops_per_segment(s: int, c1: int, c2: int, k: int) -> float:
    """Flops of a static rank-k layer: (X U) V."""
    return 2 * s * k * (c1 + c2)


def flops_matched_rank(s: int, c1: int, c2: int, k: int, r: int) -> int:
    """The largest static rank k' (a multiple of 8) whose flops do not exceed
    DyRA's at (k, r)."""
    kp = int(dyra_flops_per_segment(s, c1, c2, k, r) // (2 * s * (c1 + c2)))
    return kp // 8 * 8


def _fro_rel(a, ref):
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (d if d > 0 else 1.0))


def run_workload(w, segments: int, device="cuda", eps: float = 1e-6, input_aware: bool = True) -> dict:
    import torch
    if w.kind != synth.KIND_LOWRANK:
        raise ValueError("the E.4 static baseline is low-rank; run low-rank workloads")
    B = min(segments, w.B)
    n = B * w.s
    t0 = time.perf_counter()
    inp = synth.make_inputs(w, n_rows=n)
    X, Wm, bias = inp.X, inp.W, inp.bias
    spec = D.spec_of(w)
    f = D.prepare(Wm, spec)
    rnd = lambda a: synth.round_storage(a, w.dtype)
    W_hat = rnd(f["U"]) @ rnd(f["V"])               # the static branch as the device stores it
    W_res = Wm - W_hat
    exact = X @ Wm + (bias if bias is not None else 0.0)
    Xd = D.to_device(X, w.dtype, device)
    # E.3: t = 1, 1.5, 2 on the device
    e3 = {"t": [1.0, 1.5, 2.0], "residual_rel_err": [], "output_rel_err": []}
    seg_opt = []
    for b in range(B):
        rows = slice(b * w.s, (b + 1) * w.s)
        sv = np.linalg.svd(X[rows] @ W_res, compute_uv=False)
        seg_opt.append(float(np.sqrt(np.sum(sv[w.r:] ** 2) / np.sum(sv ** 2))))
    Ys = {}
    for h in (2, 3, 4):
        layer = D.DyraLayer(spec, f, w.dtype, bias=bias, device=device, eps=eps, half_steps=h)
        Y = layer.forward(Xd, B, w.s)
        torch.cuda.synchronize()
        Yh = Y.float().cpu().numpy().astype(np.float64)
        Ys[h] = Yh
        errs = []
        for b in range(B):
            rows = slice(b * w.s, (b + 1) * w.s)
            res = X[rows] @ W_res
            errs.append(float(np.linalg.norm(exact[rows] - Yh[rows]) / np.linalg.norm(res)))
        e3["residual_rel_err"].append(float(np.mean(errs)))
        e3["output_rel_err"].append(_fro_rel(Yh, exact))
    e3["optimal_rank_r_rel_err"] = float(np.mean(seg_opt))
    e3["static_residual_rel_err"] = 1.0
    # E.4: the FLOPs-matched static low-rank layer, (X U') V' + b on the device
    kp = flops_matched_rank(w.s, w.c1, w.c2, w.k, w.r)
    fs = D.prepare(Wm, D.make_spec(synth.KIND_LOWRANK, w.c1, w.c2, 8, k=kp))
    Ut = D.to_device(np.ascontiguousarray(rnd(fs["U"]).T), w.dtype, device)      # k' x c1
    Vt = D.to_device(np.ascontiguousarray(rnd(fs["V"]).T), w.dtype, device)      # c2 x k'
    T = torch.empty((n, kp), dtype=D.torch_dtype(w.dtype), device=device)
    Yst = torch.empty((n, w.c2), dtype=D.torch_dtype(w.dtype), device=device)
    bd = None if bias is None else D.to_device(bias, w.dtype, device)
    D.dense_ref(Xd, Ut, None, T, w.dtype)
    D.dense_ref(T, Vt, bd, Yst, w.dtype)
    torch.cuda.synchronize()
    Ystat = Yst.float().cpu().numpy().astype(np.float64)
    e4 = {"dyra_k": w.k, "dyra_r": w.r, "static_k_prime": kp,
          "dyra_gflop_per_segment": round(dyra_flops_per_segment(w.s, w.c1, w.c2, w.k, w.r) / 1e9, 4),
          "static_gflop_per_segment": round(static_flops_per_segment(w.s, w.c1, w.c2, kp) / 1e9, 4),
          "dyra_output_rel_err": e3["output_rel_err"][0],
          "static_output_rel_err": _fro_rel(Ystat, exact),
          "static_rank_k_output_rel_err": _fro_rel(X @ W_hat + (bias if bias is not None else 0.0), exact)}
    # input-aware static start (same k, r): calibration rows from an
    # independent stream of the workload's input law, so the measured
    # segments are held out
    ia = {}
    if input_aware:
        n_cal = max(2 * w.c1, 2048)
        Xc = synth.make_calibration(w, n_cal)
        for mode_name, mode in D.INPUT_AWARE.items():
            fi = D.prepare_input_aware(Wm, spec, Xc, mode)
            layer = D.DyraLayer(spec, fi, w.dtype, bias=bias, device=device, eps=eps)
            Y = layer.forward(Xd, B, w.s)
            torch.cuda.synchronize()
            Wh_i = rnd(fi["U"]) @ rnd(fi["V"])
            ia[mode_name] = {"calibration_rows": n_cal,
                             "dyra_output_rel_err": _fro_rel(Y.float().cpu().numpy().astype(np.float64), exact),
                             "static_output_rel_err": _fro_rel(X @ Wh_i + (bias if bias is not None else 0.0),
                                                               exact)}
    return {"workload": w.name, "segments": B, "tokens_per_segment": w.s, "c1": w.c1, "c2": w.c2,
            "dtype": "bf16" if w.dtype == synth.DT_BF16 else "fp32", "E3": e3, "E4": e4,
            "input_aware": ia, "seconds": round(time.perf_counter() - t0, 1)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workloads", default="vitb_fc1,vitl_fc1,vitl_fc2")
    ap.add_argument("--segments", type=int, default=4, help="segments of each workload measured (bounds host time)")
    args = ap.parse_args(argv)
    D.lib()
    for name in args.workloads.split(","):
        print(json.dumps(run_workload(synth.WORKLOADS[name], args.segments)), flush=True)


if __name__ == "__main__":
    sys.exit(main())
