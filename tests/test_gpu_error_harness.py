"""The error harness (E.3 ALS convergence, E.4 FLOPs-matched static baseline)
on a small synthetic layer: its device-measured ALS errors agree with the
float64 oracle's ALS on the same stored factors, respect the Eckart-Young
bound, do not grow with t, and its static baseline's error agrees with the
float64 product of the same stored factors."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import error_harness as H
from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O

from gpu_cases import log

pytestmark = pytest.mark.gpu


def test_harness_against_the_oracle():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w = synth.scaled(synth.WORKLOADS["vitl_fc1"], name="harness_small", B=3, s=257, c1=256, c2=512, k=64, r=16)
    res = H.run_workload(w, segments=3)
    log(f"  harness: {res}")
    e3 = res["E3"]
    # the oracle's ALS on the device's stored factors
    inp = synth.make_inputs(w)
    f = D.prepare(inp.W, D.spec_of(w))
    rnd = synth.round_bf16
    W_hat = rnd(f["U"]) @ rnd(f["V"])
    W_res_dev = rnd(f["Wres"])
    for i, t in enumerate((1.0, 1.5, 2.0)):
        errs = []
        for b in range(w.B):
            Xb = inp.X[b * w.s:(b + 1) * w.s]
            L, R = O.als(Xb, W_res_dev, f["R0"], t, 1e-6, P=rnd(f["P"]))
            target = Xb @ (inp.W - W_hat)
            errs.append(np.linalg.norm(target - L @ R) / np.linalg.norm(target))
        log(f"  t = {t}: device {e3['residual_rel_err'][i]:.4f} oracle {np.mean(errs):.4f}")
        assert abs(e3["residual_rel_err"][i] - np.mean(errs)) <= 0.02
        assert e3["residual_rel_err"][i] >= e3["optimal_rank_r_rel_err"] * 0.98
    r = e3["residual_rel_err"]
    assert r[1] <= r[0] + 0.01 and r[2] <= r[1] + 0.01
    # static baseline: the device's (X U') V' + b against float64 with the same stored factors
    e4 = res["E4"]
    fs = D.prepare(inp.W, D.make_spec(synth.KIND_LOWRANK, w.c1, w.c2, 8, k=e4["static_k_prime"]))
    exact = inp.X @ inp.W + inp.bias
    ystat = inp.X @ rnd(fs["U"]) @ rnd(fs["V"]) + inp.bias
    want = O.rel_fro(ystat, exact)
    assert abs(e4["static_output_rel_err"] - want) <= 0.01 * want + 2e-3
