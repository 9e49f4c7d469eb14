"""Shared helpers for the GPU parity tests: build a case from the seeded
generator, prepare it with the oracle, run the library on the GPU through the
C-ABI and compare with the oracle forward on the same storage-rounded inputs
and factors."""
from __future__ import annotations

import sys
import time

import numpy as np

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O

TOL = {synth.DT_F32: 1e-4, synth.DT_BF16: 2e-2}

# Finer checks than the whole-output ratio, so one wrong segment or output
# tile fails even where the correction L R is a few percent of Y:
#   per segment   ||dY_b|| <= TOL ||Y_b||
#   correction    ||dY_b|| <= ALPHA u ||Y_b|| + BETA ||(L R)_b||
#   elementwise   |dY| <= C_ELEM u (|X_b| |static factors| + a_b |L_b| |R_b| + |bias|)
# with dY = Y_gpu - Y_oracle and u the storage unit: bf16 rounds to nearest
# with u = 2^-8 relative; the fp32 path's unit is taken as 2^-16, a fifth of
# its 1e-4 bar (its error is accumulation and solve rounding, not storage).
# a_b = 1 + cond(L_b) s 2^-24 / u: G_b and M_b are fp32 sums over the s
# tokens of a segment (relative rounding up to s 2^-24), and the projection
# onto span(L_b) that the solve forms moves by that much times cond(L_b).
# Where u cond(L_b) > 1/4 (e.g. as many tokens as r), storing L_b in the
# storage precision alone moves the ridge-shrunk projection by about
# u cond(L_b) of the correction: such a segment is held to
# ||dY_b|| <= ALPHA u ||Y_b|| + BETA (1 + u cond(L_b)) ||(L R)_b|| instead of
# TOL, and a_b gains cond(L_b).  Dropping its correction still fails.
# ALPHA covers the output and first-stage (T) roundings, which measure about
# 0.45 u ||Y_b|| on the full-size cases (a 3x margin); BETA the correction's
# own roundings (L, M', R, each at most u relative) and the solve's, so a
# segment without its correction misses by ||(L R)_b||, ten times the
# allowance; C_ELEM bounds each element by four units of the magnitudes the
# device rounds.
UNIT = {synth.DT_F32: 2.0 ** -16, synth.DT_BF16: 2.0 ** -8}
ALPHA, BETA, C_ELEM = 1.5, 0.1, 4.0


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_prepare(w, W):
    return O.prepare(W, w.kind, w.r, k=w.k, mblk=w.mblk, nb=w.nb, rb=w.rb)


def host_factors_from_oracle(prep) -> dict:
    st = prep["static"]
    f = {"P": prep["P"], "R0": prep["R0"], "Wres": prep["W_res"], "res_sv": prep["res_sv"]}
    if prep["kind"] == O.KIND_LOWRANK:
        f.update(U=st["U"], V=st["V"])
    elif prep["kind"] == O.KIND_MONARCH:
        f.update(B1=st["B1"], B2=st["B2"])
    elif prep["kind"] == O.KIND_BLAST_DIAG:
        f.update(Ub=st["U"], Vb=st["V"], S=np.ascontiguousarray(np.diagonal(st["S"], axis1=2, axis2=3)))
    else:
        f.update(Ub=st["U"], Vb=st["V"], S=st["S"])
    return f


def rounded_prep(prep, dtype):
    """The oracle's prepared factors rounded to storage precision, i.e. the
    exact values the device plan holds."""
    rnd = lambda a: synth.round_storage(a, dtype)
    st = {k: rnd(v) for k, v in prep["static"].items() if k != "sv"}
    return dict(prep, static=st, P=rnd(prep["P"]), W_res=rnd(prep["W_res"]))


def gpu_forward(w, factors, X, bias, eps=1e-6, solver="auto", repeat=1, half_steps=2):
    import torch
    layer = D.DyraLayer(D.spec_of(w), factors, w.dtype, bias=bias, eps=eps, solver=D.SOLVERS[solver],
                        half_steps=half_steps)
    Xd = D.to_device(X, w.dtype)
    outs = []
    for _ in range(repeat):
        Y = layer.forward(Xd, w.B, w.s)
        torch.cuda.synchronize()
        outs.append(Y.float().cpu().numpy().astype(np.float64))
    status = layer.status(w.B, w.s)
    return outs, status


def _abs_factors(f):
    return {k: np.abs(v) for k, v in f.items()}


def oracle_terms(w, X, rp, bias, eps=1e-6, t=1.0, offsets=None):
    """The oracle forward split per segment into its static part, its
    correction L_b R_b and the magnitude |X_b||factors| + |L_b||R_b| + |bias|
    of the terms the GPU rounds.  Assembled from the oracle's own functions
    exactly as its forward assembles them (a CPU test checks the sum against
    the oracle forward bit for bit).  Returns (Y, corr, mag)."""
    n, c2 = X.shape[0], rp["W_res"].shape[1]
    Y = np.empty((n, c2))
    corr = np.empty((n, c2))
    mag = np.empty((n, c2))
    conds = []
    f, af = rp["static"], _abs_factors(rp["static"])
    for lo, hi in O.segment_rows(w.B, w.s, offsets):
        rows = slice(lo, hi)
        Xb = X[rows]
        base = O.static_apply(rp["kind"], Xb, f)
        L, R = O.als(Xb, rp["W_res"], rp["R0"], t, eps, P=rp["P"] if t >= 1 else None)
        corr[rows] = L @ R
        Y[rows] = base + corr[rows]
        sv = np.linalg.svd(L, compute_uv=False)
        cond = min(sv[0] / sv[-1], 1e12) if sv[-1] > 0 else 1e12
        conds.append(cond)
        amp = 1.0 + cond * (hi - lo) * 2.0 ** -24 / UNIT[w.dtype]
        if UNIT[w.dtype] * cond > 0.25:
            amp += cond
        mag[rows] = O.static_apply(rp["kind"], np.abs(Xb), af) + amp * (np.abs(L) @ np.abs(R))
    if bias is not None:
        Y += bias[None, :]
        mag += np.abs(bias)[None, :]
    return Y, corr, mag, conds


def parity_report(w, Yg, terms, tol=None, alpha=ALPHA, beta=BETA, c_elem=C_ELEM, offsets=None):
    """Every check above on a GPU output; returns (metrics, failures)."""
    Y, corr, mag, conds = terms
    tol = TOL[w.dtype] if tol is None else tol
    u = UNIT[w.dtype]
    d = Yg - Y
    m = {"rel_fro": O.rel_fro(Yg, Y), "seg_rel_max": 0.0, "corr_rel_max": 0.0, "corr_bound_ratio_max": 0.0,
         "corr_share": float(np.linalg.norm(corr) / max(np.linalg.norm(Y), 1e-300))}
    fails = []
    if not np.all(np.isfinite(Yg)):
        fails.append("non-finite output")
    if m["rel_fro"] > tol:
        fails.append(f"rel_fro {m['rel_fro']:.3e} > {tol}")
    for b, (lo, hi) in enumerate(O.segment_rows(w.B, w.s, offsets)):
        rows = slice(lo, hi)
        db, yb, cb = np.linalg.norm(d[rows]), np.linalg.norm(Y[rows]), np.linalg.norm(corr[rows])
        sr = db / max(yb, 1e-300)
        ill = u * conds[b] > 0.25
        bound = alpha * u * yb + beta * (1.0 + (u * conds[b] if ill else 0.0)) * cb
        m["seg_rel_max"] = max(m["seg_rel_max"], sr)
        if cb > 0:
            m["corr_rel_max"] = max(m["corr_rel_max"], db / cb)
        m["corr_bound_ratio_max"] = max(m["corr_bound_ratio_max"], db / max(bound, 1e-300))
        if ill:
            m["ill_conditioned_segments"] = m.get("ill_conditioned_segments", 0) + 1
        elif sr > tol:
            fails.append(f"segment {b}: rel_fro {sr:.3e} > {tol}")
        if db > bound:
            fails.append(f"segment {b}: ||dY|| {db:.3e} > {alpha} u ||Y_b|| + {beta} ||(LR)_b|| = {bound:.3e}")
    ratio = np.abs(d) / (c_elem * u * mag + 1e-300)
    m["elem_ratio_max"] = float(np.max(ratio)) if ratio.size else 0.0
    if m["elem_ratio_max"] > 1.0:
        i, j = np.unravel_index(np.argmax(ratio), ratio.shape)
        fails.append(f"element ({i}, {j}): |dY| {abs(d[i, j]):.3e} > {c_elem} u mag = {c_elem * u * mag[i, j]:.3e}")
    return m, fails


def gpu_forward_varlen(w, factors, X, bias, offsets, eps=1e-6, solver="auto", half_steps=2):
    """The forward over ragged segments (row offsets) through dyra_forward_varlen_als."""
    import torch
    layer = D.DyraLayer(D.spec_of(w), factors, w.dtype, bias=bias, eps=eps, solver=D.SOLVERS[solver],
                        half_steps=half_steps)
    Y, st = layer.forward_varlen(D.to_device(X, w.dtype), offsets)
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64), st.cpu().numpy()


def run_same_factor_case(w, eps=1e-6, solver="auto", tol=None, inputs=None, prep=None, half_steps=2,
                         alpha=ALPHA, beta=BETA, c_elem=C_ELEM, offsets=None):
    """Same-factor parity: GPU forward vs oracle forward on identical inputs
    and identical (rounded) factors, with t = half_steps / 2 ALS iterations,
    judged by parity_report.  Returns (err, status, Y_gpu, Y_oracle)."""
    t0 = time.time()
    inp = inputs if inputs is not None else synth.make_inputs(w)
    if prep is None:
        prep = oracle_prepare(w, inp.W)
    rp = rounded_prep(prep, w.dtype)
    terms = oracle_terms(w, inp.X, rp, inp.bias, eps=eps, t=half_steps / 2, offsets=offsets)
    t1 = time.time()
    if offsets is None:
        (Yg,), status = gpu_forward(w, host_factors_from_oracle(prep), inp.X, inp.bias, eps=eps, solver=solver,
                                    half_steps=half_steps)
    else:
        Yg, status = gpu_forward_varlen(w, host_factors_from_oracle(prep), inp.X, inp.bias, offsets, eps=eps,
                                        solver=solver, half_steps=half_steps)
    m, fails = parity_report(w, Yg, terms, tol=tol, alpha=alpha, beta=beta, c_elem=c_elem, offsets=offsets)
    log(f"  case {w.name} B={w.B} s={w.s} c1={w.c1} c2={w.c2} r={w.r} k={w.k} dtype={w.dtype} "
        f"solver={solver} t={half_steps / 2}: rel_fro={m['rel_fro']:.3e} seg_max={m['seg_rel_max']:.3e} "
        f"corr_rel_max={m['corr_rel_max']:.3e} (LR share {m['corr_share']:.3f}, bound ratio "
        f"{m['corr_bound_ratio_max']:.2f}) elem_ratio={m['elem_ratio_max']:.2f} "
        f"status={np.unique(status).tolist()} (oracle {t1 - t0:.1f}s, gpu {time.time() - t1:.1f}s)")
    assert not fails, "; ".join(fails[:5])
    return m["rel_fro"], status, Yg, terms[0]
