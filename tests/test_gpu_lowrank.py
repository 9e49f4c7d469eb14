"""GPU parity of the low-rank DyRA forward against the float64 oracle, through
the C-ABI.  Bars: relative Frobenius error <= 1e-4 (fp32) / 2e-2 (bf16 with
fp32 accumulation) on the same seeded inputs and the same storage-rounded
factors.  Run on an MI355X: pytest -m gpu."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O

from gpu_cases import (TOL, gpu_forward, host_factors_from_oracle, log, oracle_prepare, rounded_prep,
                       run_same_factor_case)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
sc = synth.scaled


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    D.lib()


SMALL = [
    W["tiny_fp32"],
    sc(W["vitb_fc1"], name="ragged_bf16", B=3, s=77, c1=192, c2=200, k=24, r=16),
    sc(W["vitb_fc1"], name="ragged_fp32", B=3, s=77, c1=192, c2=200, k=24, r=16, dtype=synth.DT_F32),
    sc(W["vitb_fc1"], name="one_small_tile", B=1, s=20, c1=64, c2=64, k=8, r=8),
    sc(W["vitb_fc1"], name="many_short_segments", B=37, s=13, c1=128, c2=136, k=16, r=8),
    sc(W["vitb_fc1"], name="wide_k", B=2, s=300, c1=512, c2=256, k=200, r=56),
    # right factor split over K: 3 slices of 384, 384 and 232 (ragged), on a
    # 200 x 32 output (ragged 128 x 128 tiles)
    sc(W["vitb_fc1"], name="split_k_right_factor", B=2, s=100, c1=1000, c2=200, k=64, r=16),
    # M' = Ginv M with four 16-row blocks per wave (32 segments x 64 column
    # tiles) and r = 56 (the last block ragged); right factor in 4 K slices
    sc(W["vitb_fc1"], name="apply_four_blocks_ragged_r", B=32, s=64, c1=4096, c2=256, k=64, r=56),
    # r = 40: reduction chunks past r load as zeros in the load-all path
    sc(W["vitb_fc1"], name="apply_r40", B=3, s=77, c1=192, c2=200, k=24, r=40),
    sc(W["vitl_fc1"], name="r128_ns", B=2, s=300, c1=256, c2=384, k=64, r=128, solver="ns"),
    # fp32 storage through Newton-Schulz: split-precision phase, then the
    # fp32 polish to its floor (the fp32 bar applies)
    sc(W["vitb_fc1"], name="ragged_fp32_ns", B=3, s=77, c1=192, c2=200, k=24, r=16, dtype=synth.DT_F32,
       solver="ns"),
    sc(W["vitl_fc1"], name="r128_ns_fp32", B=2, s=300, c1=256, c2=384, k=64, r=128, dtype=synth.DT_F32,
       solver="ns"),
    # k + r = 320: the 160 x 320 first-stage tile, ragged in rows
    sc(W["vitl_fc1"], name="wide_first_stage_tile", B=3, s=150, c1=384, c2=384, k=256, r=64),
    # bf16 without bias: the persistent output kernel's zero-addend variant
    sc(W["vitb_fc1"], name="ragged_bf16_nobias", B=3, s=77, c1=192, c2=200, k=24, r=16, bias=False),
    # about 4.5 output tiles per persistent workgroup, a segment boundary inside tiles
    sc(W["vitl_fc1"], name="persistent_several_tiles", B=10, s=900, c1=256, c2=4096, k=64, r=32),
    sc(W["vitl_fc1"], name="persistent_several_tiles_nobias", B=10, s=900, c1=256, c2=4096, k=64, r=32,
       bias=False),
    # r = 64, k = 256 / 128, long segments: several 256 x 128 output tiles per
    # persistent workgroup with segment boundaries inside tiles and a ragged
    # last row block (with and without bias); then ragged columns (c2 = 1000)
    sc(W["vitl_fc1"], name="a_stationary_k256", B=7, s=1029, c1=512, c2=4096, k=256, r=64),
    sc(W["vitl_fc1"], name="a_stationary_k128_nobias", B=9, s=700, c1=256, c2=4096, k=128, r=64, bias=False),
    sc(W["vitl_fc1"], name="a_stationary_ragged_cols", B=2, s=600, c1=384, c2=1000, k=256, r=64),
    # first-stage Gram partials: 170-token segments, so nearly every 160-row
    # tile meets two segments (both partial slots in use)
    sc(W["vitl_fc1"], name="first_stage_gram_short_segments", B=20, s=170, c1=384, c2=512, k=256, r=64),
    # the right factor R^T (4096 x 40 * 64) has 320 tiles of 256 x 128, more
    # than one per persistent workgroup of its no-residual-part GEMM: each
    # workgroup's later tiles must get their own operands (they came out of
    # zero-filled loads when the loaders did not leave an empty L R part)
    sc(W["vitl_fc1"], name="right_factor_several_tiles", B=40, s=160, c1=256, c2=4096, k=64, r=64),
    # few (segment, column strip) pairs: the M strips split their tokens
    # into parts whose fp32 partials a second launch adds (4 parts here)
    sc(W["vitl_fc1"], name="token_split_long_segments", B=2, s=2100, c1=512, c2=512, k=64, r=64),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_cases(w):
    run_same_factor_case(w, solver=w.solver)


@pytest.mark.parametrize("solver", ["chol", "ns"])
def test_solver_choice_r64(solver):
    w = sc(W["vitl_fc1"], name=f"r64_{solver}", B=4, s=257, c1=256, c2=512, k=64, r=64)
    err, status, _, _ = run_same_factor_case(w, solver=solver)
    assert np.all(status == D.SOLVE_OK)


def test_segment_shorter_than_rank():
    """s < r: L_b is rank deficient, G_b singular; the ridge keeps it SPD."""
    w = sc(W["vitb_fc1"], name="s_lt_r", B=6, s=5, c1=128, c2=128, k=16, r=16)
    run_same_factor_case(w, eps=1e-3)


@pytest.mark.parametrize("name", ["vitb_fc1", "vitl_fc1", "vitl_fc2"])
def test_full_size(name):
    w = W[name]
    err, status, _, _ = run_same_factor_case(w)
    assert np.all(status == D.SOLVE_OK)


def test_full_size_larger_batch():
    """ViT-L fc1 at 40 images (41160 tokens): more first-stage tiles than
    CUs (a second round), 40 segments in the XCD-grouped token reduction,
    and a right factor R^T with 320 tiles of 256 x 128, more than one per
    persistent workgroup."""
    w = sc(W["vitl_fc1"], name="vitl_fc1_b40", B=40)
    err, status, _, _ = run_same_factor_case(w)
    assert np.all(status == D.SOLVE_OK)


def test_zero_residual_gives_static_output_and_zero_status():
    """W of exact rank k: P = W_res = 0, so G_b = 0, status ZERO and
    Y = X W_hat + bias."""
    rng = np.random.default_rng(11)
    w = sc(W["vitb_fc1"], name="zero_res", B=2, s=64, c1=128, c2=128, k=16, r=8)
    inp = synth.make_inputs(w)
    U = synth.haar_columns(rng.standard_normal((128, 16)))
    V = synth.haar_columns(rng.standard_normal((128, 16)))
    Wk = synth.round_bf16((U * np.linspace(1, 0.5, 16)) @ V.T)
    prep = oracle_prepare(w, Wk)
    prep["W_res"] = np.zeros_like(prep["W_res"])
    prep["P"] = np.zeros_like(prep["P"])
    inp2 = synth.Inputs(X=inp.X, W=Wk, bias=inp.bias, W_exact=Wk, spectrum=None)
    err, status, Yg, Y_or = run_same_factor_case(w, inputs=inp2, prep=prep)
    assert np.all(status == D.SOLVE_ZERO)
    rp = rounded_prep(prep, w.dtype)
    static = O.static_apply(w.kind, inp.X, rp["static"]) + inp.bias
    assert O.rel_fro(Yg, static) <= TOL[w.dtype]


def test_bitwise_deterministic():
    w = sc(W["vitb_fc1"], name="det", B=3, s=100, c1=256, c2=256, k=32, r=16)
    inp = synth.make_inputs(w)
    prep = oracle_prepare(w, inp.W)
    from gpu_cases import host_factors_from_oracle
    outs, _ = gpu_forward(w, host_factors_from_oracle(prep), inp.X, inp.bias, repeat=3)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("name", ["tiny_fp32", "vitl_fc1"])
def test_end_to_end_library_prepare(name):
    """End-to-end: the library's own host prepare + GPU forward vs the oracle's
    prepare + forward (both from the same W)."""
    w = W[name]
    inp = synth.make_inputs(w)
    f = D.prepare(inp.W, D.spec_of(w))
    (Yg,), status = gpu_forward(w, f, inp.X, inp.bias)
    prep = oracle_prepare(w, inp.W)
    Y_or = O.forward(inp.X, prep, inp.bias, w.B, w.s, eps=1e-6)
    err = O.rel_fro(Yg, Y_or)
    log(f"  end-to-end {name}: rel_fro={err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", [synth.DT_F32, synth.DT_BF16])
def test_dense_ref(dtype):
    import torch
    rng = np.random.default_rng(5)
    n, c1, c2 = 300, 264, 200
    X = synth.round_storage(rng.standard_normal((n, c1)), dtype)
    Wm = synth.round_storage(rng.standard_normal((c1, c2)) / np.sqrt(c1), dtype)
    b = synth.round_storage(rng.standard_normal(c2), dtype)
    Xd, Wt, bd = D.to_device(X, dtype), D.to_device(Wm.T.copy(), dtype), D.to_device(b, dtype)
    Y = torch.empty((n, c2), dtype=D.torch_dtype(dtype), device="cuda")
    D.dense_ref(Xd, Wt, bd, Y, dtype)
    torch.cuda.synchronize()
    ref = X @ Wm + b
    err = O.rel_fro(Y.float().cpu().numpy().astype(float), ref)
    # fp32: accumulation rounding only; bf16: plus the output rounding (2^-9)
    assert err <= (1e-5 if dtype == synth.DT_F32 else 4e-3), err


# ---------------------------------------------------------------------------
# the Cholesky route (DYRA_SOLVER_CHOL): factor, triangular inverse, W^T W
# ---------------------------------------------------------------------------

CHOL = [sc(W["vitb_fc1"], name=f"chol_r{r}", B=3, s=150, c1=256, c2=264, k=32, r=r, solver="chol")
        for r in (8, 16, 32, 56, 64)] + [
    sc(W["vitl_fc1"], name="chol_r128", B=2, s=300, c1=256, c2=384, k=64, r=128, solver="chol"),
    sc(W["vitb_fc1"], name="chol_fp32_r16", B=3, s=77, c1=192, c2=200, k=24, r=16, dtype=synth.DT_F32,
       solver="chol"),
    sc(W["vitl_fc1"], name="chol_fp32_r128", B=2, s=300, c1=256, c2=384, k=64, r=128, dtype=synth.DT_F32,
       solver="chol"),
]


@pytest.mark.parametrize("w", CHOL, ids=lambda w: w.name)
def test_cholesky_route(w):
    err, status, _, _ = run_same_factor_case(w, solver="chol")
    assert np.all(status == D.SOLVE_OK)


def test_cholesky_route_full_size_vitl():
    err, status, _, _ = run_same_factor_case(W["vitl_fc1"], solver="chol")
    assert np.all(status == D.SOLVE_OK)


# ---------------------------------------------------------------------------
# no ridge (eps = 0): a numerically singular G_b drops the correction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("solver", ["auto", "chol"])
@pytest.mark.parametrize("dtype", [synth.DT_BF16, synth.DT_F32])
def test_unridged_segment_shorter_than_rank_drops_the_correction(solver, dtype):
    """s < r at eps = 0: G_b has rank s, a pivot falls below 2^-16 of its
    diagonal, the status is NOT_SPD and Y_b = X_b W_hat + bias, as in the
    oracle's reading of an unridged singular system."""
    w = sc(W["vitb_fc1"], name=f"s_lt_r_eps0_{solver}", B=6, s=5, c1=128, c2=128, k=16, r=16, dtype=dtype)
    err, status, Yg, Y_or = run_same_factor_case(w, eps=0.0, solver=solver)
    assert np.all(status == D.SOLVE_NOT_SPD), status
    inp = synth.make_inputs(w)
    rp = rounded_prep(oracle_prepare(w, inp.W), w.dtype)
    static = O.static_apply(w.kind, inp.X, rp["static"]) + inp.bias
    np.testing.assert_array_equal(Y_or, static)


@pytest.mark.parametrize("solver", ["auto", "chol"])
def test_unridged_full_rank_segments_solve(solver):
    w = sc(W["vitb_fc1"], name=f"eps0_full_rank_{solver}", B=3, s=200, c1=256, c2=264, k=32, r=32)
    err, status, _, _ = run_same_factor_case(w, eps=0.0, solver=solver)
    assert np.all(status == D.SOLVE_OK)


def test_non_finite_input_stays_in_its_segment():
    """A NaN in one token of segment 1: that segment's trace is NaN, its
    status NOT_SPD and R_1 = 0, so only the NaN token's own output row is
    non-finite and the segment's other rows are the static branch
    X_b W_hat + bias; every other segment's output is bit for bit that of
    the clean input (tiles shared across the segment boundary included)."""
    import torch  # noqa: F401
    w = sc(W["vitb_fc1"], name="nan_segment", B=4, s=100, c1=256, c2=264, k=32, r=16)
    inp = synth.make_inputs(w)
    prep = oracle_prepare(w, inp.W)
    f = host_factors_from_oracle(prep)
    (clean,), st_clean = gpu_forward(w, f, inp.X, inp.bias)
    Xn = inp.X.copy()
    Xn[150, 7] = np.nan
    (dirty,), st = gpu_forward(w, f, Xn, inp.bias)
    seg1 = dirty[100:200]
    bad_rows = np.where(~np.isfinite(seg1).all(axis=1))[0].tolist()
    log(f"  nan_segment: status clean {st_clean.tolist()} dirty {st.tolist()}; non-finite rows of segment 1: "
        f"{bad_rows}")
    assert st_clean.tolist() == [D.SOLVE_OK] * 4
    assert st.tolist() == [D.SOLVE_OK, D.SOLVE_NOT_SPD, D.SOLVE_OK, D.SOLVE_OK]
    assert bad_rows == [50]
    rp = rounded_prep(prep, w.dtype)
    keep = np.r_[100:150, 151:200]
    static = O.static_apply(w.kind, inp.X[keep], rp["static"]) + inp.bias
    assert O.rel_fro(dirty[keep], static) <= TOL[w.dtype]
    for b in (0, 2, 3):
        np.testing.assert_array_equal(dirty[b * 100:(b + 1) * 100], clean[b * 100:(b + 1) * 100])


# ---------------------------------------------------------------------------
# input-aware static start: a prepare-only variant, the forward is unchanged
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [D.INPUT_AWARE_DIAG, D.INPUT_AWARE_CHOL])
def test_input_aware_start(mode):
    """Same-factor parity with the oracle's input-aware prepare, and the
    library's own input-aware prepare end to end against the oracle's."""
    w = sc(W["vitl_fc1"], name=f"input_aware_{mode}", B=4, s=257, c1=256, c2=512, k=64, r=32)
    inp = synth.make_inputs(w)
    Xc = synth.make_calibration(w, 1024)
    prep = O.prepare(inp.W, w.kind, w.r, k=w.k, calib=(Xc, mode))
    err, status, _, _ = run_same_factor_case(w, inputs=inp, prep=prep)
    assert np.all(status == D.SOLVE_OK)
    f = D.prepare_input_aware(inp.W, D.spec_of(w), Xc, mode)
    (Yg,), status = gpu_forward(w, f, inp.X, inp.bias)
    e2e = O.rel_fro(Yg, O.forward(inp.X, prep, inp.bias, w.B, w.s, eps=1e-6))
    log(f"  input-aware mode {mode}: end to end rel_fro {e2e:.3e}")
    assert e2e <= TOL[w.dtype] and np.all(status == D.SOLVE_OK)
