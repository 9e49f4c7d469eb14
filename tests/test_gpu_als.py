"""GPU parity of the forward with more than one ALS iteration (t = 1.5, 2)
against the float64 oracle's ALS, through the C-ABI (dyra_forward_als), and
the property the pages state for more iterations: the approximation error
does not grow with t.  Run on an MI355X: pytest -m gpu."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O

from gpu_cases import TOL, gpu_forward, host_factors_from_oracle, log, oracle_prepare, run_same_factor_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
sc = synth.scaled


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    D.lib()


CASES = [
    sc(W["vitb_fc1"], name="als_ragged", B=3, s=77, c1=192, c2=200, k=24, r=16),
    sc(W["vitl_fc1"], name="als_r64", B=4, s=257, c1=256, c2=512, k=64, r=64),
    sc(W["vitl_fc1"], name="als_r128", B=2, s=300, c1=256, c2=384, k=64, r=128),
    sc(W["vitb_fc1"], name="als_short_segments", B=9, s=11, c1=128, c2=136, k=16, r=8),
]


# fp32 storage (low-rank, the one structure with fp32): the left step on
# the fp32 token reduction, the sweep and the engine GEMM; the fp32 bar
CASES_F32 = [
    W["tiny_fp32"],
    sc(W["vitb_fc1"], name="als_ragged_fp32", B=3, s=77, c1=192, c2=200, k=24, r=16, dtype=synth.DT_F32),
    sc(W["vitl_fc1"], name="als_r64_fp32", B=4, s=257, c1=256, c2=512, k=64, r=64, dtype=synth.DT_F32),
]


@pytest.mark.parametrize("half_steps", [3, 4])
@pytest.mark.parametrize("w", CASES + CASES_F32, ids=lambda w: w.name)
def test_als_parity(w, half_steps):
    err, status, _, _ = run_same_factor_case(w, half_steps=half_steps)
    assert np.all(status == D.SOLVE_OK)


# the structured static branches: the left step is the same (it does not
# involve W_hat); only where L sits in the first-stage output differs
STRUCTURED = [
    sc(W["monarch"], name="als_monarch", B=3, s=77),
    sc(W["lm_blast"], name="als_blast", B=2, s=200, c1=512, c2=1536, nb=4, rb=32, r=32, solver="auto"),
    sc(W["lm_blast_diag"], name="als_blast_diag", B=2, s=200, c1=512, c2=1536, nb=4, rb=32, r=32,
       solver="auto"),
]


@pytest.mark.parametrize("half_steps", [3, 4])
@pytest.mark.parametrize("w", STRUCTURED, ids=lambda w: w.name)
def test_als_structured(w, half_steps):
    err, status, _, _ = run_same_factor_case(w, half_steps=half_steps)
    assert np.all(status == D.SOLVE_OK)


@pytest.mark.parametrize("half_steps", [3, 4])
def test_als_full_size_vitl(half_steps):
    run_same_factor_case(W["vitl_fc1"], half_steps=half_steps)


def test_error_does_not_grow_with_t():
    """||X W + bias - Y_t||_F for t = 1, 1.5, 2 on the GPU: non-increasing up to
    the bf16 storage of the output (slack 2^-8 relative to ||X W||)."""
    w = sc(W["vitl_fc1"], name="als_monotone", B=4, s=257, c1=256, c2=512, k=64, r=64)
    inp = synth.make_inputs(w)
    prep = oracle_prepare(w, inp.W)
    f = host_factors_from_oracle(prep)
    exact = inp.X @ synth.round_storage(inp.W, w.dtype) + inp.bias
    errs = []
    for h in (2, 3, 4):
        (Yg,), status = gpu_forward(w, f, inp.X, inp.bias, half_steps=h)
        assert np.all(status == D.SOLVE_OK)
        errs.append(np.linalg.norm(Yg - exact))
    slack = 2.0 ** -8 * np.linalg.norm(exact)
    log(f"  ||XW - Y_t||_F for t = 1, 1.5, 2: {[f'{e:.4e}' for e in errs]} (slack {slack:.2e})")
    assert errs[1] <= errs[0] + slack and errs[2] <= errs[1] + slack
