"""Pins of the float64 oracle against facts the DyRA pages and linear algebra fix.

Each test names the passage it follows.  Pages: [P2] the paperlayer.ai
section summary of arXiv 2610.02882; [P5] the nanless.github.io DyRA digest.
These run on the CPU only.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg as sla

from oracle import dyra_oracle as O
from input_adaptive_rank_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _power_law_w(rng, c1, c2, alpha=0.5):
    m = min(c1, c2)
    U = synth.haar_columns(rng.standard_normal((c1, m)))
    V = synth.haar_columns(rng.standard_normal((c2, m)))
    s = np.arange(1, m + 1, dtype=float) ** -alpha
    return (U * s) @ V.T, U, s, V


def _aniso_x(rng, n, c1):
    sig = synth.channel_scales(c1, rng.choice(c1, 2, replace=False))
    return rng.standard_normal((n, c1)) * sig


def _prep_lowrank(W, k, r):
    return O.prepare(W, O.KIND_LOWRANK, r, k=k)


# ---------------------------------------------------------------------------
# hand-derived worked examples ([P5] split + objective + one-step form)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden()["dyra_lowrank"], ids=lambda c: c["name"])
def test_hand_worked_dyra(case):
    X = np.array(case["X"], float)
    W = np.array(case["W"], float)
    B = case.get("B", 1)
    s = case.get("s", X.shape[0])
    bias = None if case["bias"] is None else np.array(case["bias"], float)
    prep = _prep_lowrank(W, case["k"], case["r"])
    Y = O.forward(X, prep, bias, B, s, eps=case["eps"])
    np.testing.assert_allclose(Y, np.array(case["Y"], float), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", _golden()["monarch"], ids=lambda c: c["name"])
def test_hand_worked_monarch(case):
    f = {"B1": np.array(case["B1"], float), "B2": np.array(case["B2"], float)}
    np.testing.assert_array_equal(O.monarch_dense(f), np.array(case["W_hat"], float))
    X = np.array(case["X"], float)
    np.testing.assert_allclose(O.monarch_apply(X, f), np.array(case["Y"], float), atol=1e-12)


@pytest.mark.parametrize("case", _golden()["blast"], ids=lambda c: c["name"])
def test_hand_worked_blast(case):
    f = {k: np.array(case[k], float) for k in ("U", "V", "S")}
    np.testing.assert_allclose(O.blast_dense(f), np.array(case["W_hat"], float), atol=1e-12)
    X = np.array(case["X"], float)
    np.testing.assert_allclose(O.blast_apply(X, f), np.array(case["Y"], float), atol=1e-12)


@pytest.mark.parametrize("case", _golden()["als"], ids=lambda c: c["name"])
def test_hand_worked_als(case):
    """More ALS half-steps on the diag3 example (t = 1.5: L, R, L; t = 2:
    L, R, L, R), values derived by hand.  The sign of R0 is free, so the
    factors are compared up to one common sign; Y is sign free."""
    X = np.array(case["X"], float)
    W = np.array(case["W"], float)
    prep = _prep_lowrank(W, case["k"], case["r"])
    Y = O.forward(X, prep, None, 1, X.shape[0], eps=case["eps"], t=case["t"])
    np.testing.assert_allclose(Y, np.array(case["Y"], float), rtol=0, atol=1e-12)
    L, R = O.als(X, prep["W_res"], prep["R0"], case["t"], case["eps"], P=prep["P"])
    for name, got in (("L", L[:, 0]), ("R", R[0])):
        if name in case:
            want = np.array(case[name], float)
            sgn = np.sign(got[np.argmax(np.abs(want))]) * np.sign(want[np.argmax(np.abs(want))])
            np.testing.assert_allclose(sgn * got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# The R update is exact least squares ([P5] objective; [P2] 2.2 ridge)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 1e-3, 0.3])
def test_right_step_is_bruteforce_least_squares(eps):
    rng = _rng(1)
    W, *_ = _power_law_w(rng, 24, 20)
    X = _aniso_x(rng, 40, 24)
    prep = _prep_lowrank(W, 6, 4)
    L = X @ prep["P"]
    R = O.right_step(X, prep["W_res"], L, eps)
    T = X @ prep["W_res"]                      # explicit residual product (tiny)
    if eps == 0:
        R_bf = np.linalg.lstsq(L, T, rcond=None)[0]
    else:
        lam = eps * np.trace(L.T @ L) / L.shape[1]
        A = np.vstack([L, np.sqrt(lam) * np.eye(L.shape[1])])
        R_bf = np.linalg.lstsq(A, np.vstack([T, np.zeros((L.shape[1], T.shape[1]))]), rcond=None)[0]
    np.testing.assert_allclose(R, R_bf, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_orthogonality_of_correction(eps):
    """L^T (X W_res - L R) = lambda R (0 at eps = 0): the correction is the
    (ridge-)projection of X W_res onto span(L)."""
    rng = _rng(2)
    W, *_ = _power_law_w(rng, 32, 48)
    X = _aniso_x(rng, 64, 32)
    prep = _prep_lowrank(W, 8, 6)
    fac = O.forward_segment_factors(X, prep["W_res"], prep["P"], eps)
    L, R = fac["L"], fac["R"]
    lhs = L.T @ (X @ prep["W_res"] - L @ R)
    np.testing.assert_allclose(lhs, fac["lam"] * R, atol=1e-10 * np.abs(L.T @ X @ prep["W_res"]).max())


def test_left_step_is_bruteforce_least_squares():
    rng = _rng(3)
    W, *_ = _power_law_w(rng, 20, 30)
    X = _aniso_x(rng, 25, 20)
    prep = _prep_lowrank(W, 5, 3)
    R = rng.standard_normal((3, 30))
    L = O.left_step(X, prep["W_res"], R, 0.0)
    T = X @ prep["W_res"]
    L_bf = np.linalg.lstsq(R.T, T.T, rcond=None)[0].T     # min ||T - L R|| over L
    np.testing.assert_allclose(L, L_bf, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("eps", [1e-3, 0.3])
def test_left_step_with_ridge_is_augmented_least_squares(eps):
    """eps > 0, r = 3: L minimises ||X W_res - L R||^2 + lambda ||L||^2 with
    lambda = eps trace(R R^T) / r, i.e. least squares on the augmented system
    [R^T; sqrt(lambda) I] L^T = [(X W_res)^T; 0] on an explicit X W_res."""
    rng = _rng(5)
    W, *_ = _power_law_w(rng, 20, 30)
    X = _aniso_x(rng, 25, 20)
    prep = _prep_lowrank(W, 5, 3)
    R = rng.standard_normal((3, 30)) * np.array([[3.0], [1.0], [0.2]])
    L = O.left_step(X, prep["W_res"], R, eps)
    T = X @ prep["W_res"]
    lam = eps * np.sum(R * R) / 3
    A = np.vstack([R.T, np.sqrt(lam) * np.eye(3)])
    L_bf = np.linalg.lstsq(A, np.vstack([T.T, np.zeros((3, T.shape[0]))]), rcond=None)[0].T
    np.testing.assert_allclose(L, L_bf, rtol=1e-9, atol=1e-12)


def test_first_left_step_uses_precomputed_projection():
    """L = X (W_res R0^T)(R0 R0^T)^-1 equals X P since R0 has orthonormal rows."""
    rng = _rng(4)
    W, *_ = _power_law_w(rng, 30, 22)
    X = _aniso_x(rng, 17, 30)
    prep = _prep_lowrank(W, 4, 5)
    np.testing.assert_allclose(prep["R0"] @ prep["R0"].T, np.eye(5), atol=1e-12)
    np.testing.assert_allclose(O.left_step(X, prep["W_res"], prep["R0"], 0.0), X @ prep["P"],
                               rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# error bounds ([P5] split equation; [P2] E.3 optimal rank-r reference)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.1])
def test_never_worse_than_static(seed, eps):
    rng = _rng(10 + seed)
    W, *_ = _power_law_w(rng, 40, 56)
    X = _aniso_x(rng, 50, 40)
    prep = _prep_lowrank(W, 10, 6)
    Y = O.forward(X, prep, None, 1, 50, eps=eps)
    exact = X @ W
    static = X @ prep["W_hat"]
    assert np.linalg.norm(exact - Y) <= np.linalg.norm(exact - static) * (1 + 1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_eckart_young_lower_bound(seed):
    rng = _rng(20 + seed)
    W, *_ = _power_law_w(rng, 36, 44)
    X = _aniso_x(rng, 60, 36)
    r = 5
    prep = _prep_lowrank(W, 8, r)
    T = X @ prep["W_res"]
    L, R = O.als(X, prep["W_res"], prep["R0"], 1.0, 0.0, P=prep["P"])
    opt = np.sqrt(np.sum(np.linalg.svd(T, compute_uv=False)[r:] ** 2))
    err = np.linalg.norm(T - L @ R)
    assert err >= opt * (1 - 1e-12)


def test_als_error_non_increasing_in_t():
    rng = _rng(30)
    W, *_ = _power_law_w(rng, 48, 40)
    X = _aniso_x(rng, 80, 48)
    prep = _prep_lowrank(W, 8, 6)
    T = X @ prep["W_res"]
    errs = []
    for t in (1.0, 1.5, 2.0, 3.0):
        L, R = O.als(X, prep["W_res"], prep["R0"], t, 0.0, P=prep["P"])
        errs.append(np.linalg.norm(T - L @ R))
    assert all(b <= a * (1 + 1e-12) for a, b in zip(errs, errs[1:]))


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.05])
def test_als_half_steps_are_stationary(eps):
    """t = 1.5 ends on a left step: (X W_res - L R) R^T = lambda_L L with
    lambda_L = eps trace(R R^T) / r for the R of the preceding right step;
    t = 2 ends on a right step: L^T (X W_res - L R) = lambda R with
    lambda = eps trace(L^T L) / r.  Both are the normal equations of the
    half-step just taken (the pages' alternating least squares)."""
    rng = _rng(31)
    W, *_ = _power_law_w(rng, 40, 36)
    X = _aniso_x(rng, 70, 40)
    r = 5
    prep = _prep_lowrank(W, 8, r)
    T = X @ prep["W_res"]
    scale = np.abs(T).max() * np.abs(prep["W_res"]).max() * 100
    L, R = O.als(X, prep["W_res"], prep["R0"], 1.5, eps, P=prep["P"])
    lam_l = eps * np.trace(R @ R.T) / r
    np.testing.assert_allclose((T - L @ R) @ R.T, lam_l * L, atol=1e-11 * scale)
    assert np.linalg.norm(L - X @ prep["P"]) > 1e-3 * np.linalg.norm(L)   # the left step moved L
    L2, R2 = O.als(X, prep["W_res"], prep["R0"], 2.0, eps, P=prep["P"])
    np.testing.assert_allclose(L2, L, atol=0)                              # same first three half-steps
    lam_r = eps * np.trace(L2.T @ L2) / r
    np.testing.assert_allclose(L2.T @ (T - L2 @ R2), lam_r * R2, atol=1e-11 * scale)


def test_als_error_strictly_decreases_on_a_generic_case():
    """On a generic input each extra half-step strictly lowers the error of
    L R against X W_res, so Y(1.5) differs from Y(1) and Y(2) from Y(1.5)."""
    rng = _rng(32)
    W, *_ = _power_law_w(rng, 48, 40)
    X = _aniso_x(rng, 80, 48)
    prep = _prep_lowrank(W, 8, 6)
    T = X @ prep["W_res"]
    errs, Ys = [], []
    for t in (1.0, 1.5, 2.0):
        L, R = O.als(X, prep["W_res"], prep["R0"], t, 1e-6, P=prep["P"])
        errs.append(np.linalg.norm(T - L @ R))
        Ys.append(O.forward(X, prep, None, 1, 80, eps=1e-6, t=t))
    assert errs[1] < errs[0] * (1 - 1e-3) and errs[2] < errs[1] * (1 - 1e-4)
    assert O.rel_fro(Ys[1], Ys[0]) > 1e-3 and O.rel_fro(Ys[2], Ys[1]) > 1e-4


# ---------------------------------------------------------------------------
# Proposition 1 ([P2] 2.3 and App. C): X^T X = I reproduces static rank k+r
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [1.0, 3.7])
def test_proposition1_isotropic_equals_rank_k_plus_r(scale):
    rng = _rng(40)
    c1, c2, k, r = 24, 30, 5, 4
    W, U, s, V = _power_law_w(rng, c1, c2)
    X = synth.orthonormal_rows_input(rng, 64, c1, scale)
    prep = _prep_lowrank(W, k, r)
    Y = O.forward(X, prep, None, 1, 64, eps=0.0)
    W_kr = (U[:, :k + r] * s[:k + r]) @ V[:, :k + r].T
    np.testing.assert_allclose(Y, X @ W_kr, atol=1e-10 * scale)


def test_proposition1_with_ridge_shrinks_by_closed_form():
    rng = _rng(41)
    c1, c2, k, r, eps = 20, 26, 4, 5, 0.05
    W, U, s, V = _power_law_w(rng, c1, c2)
    X = synth.orthonormal_rows_input(rng, 40, c1, 2.0)
    prep = _prep_lowrank(W, k, r)
    Y = O.forward(X, prep, None, 1, 40, eps=eps)
    sr = s[k:k + r]
    lam = eps * np.mean(sr ** 2)
    D = sr ** 2 / (sr ** 2 + lam)
    W_eff = (U[:, :k] * s[:k]) @ V[:, :k].T + (U[:, k:k + r] * (sr * D)) @ V[:, k:k + r].T
    np.testing.assert_allclose(Y, X @ W_eff, atol=1e-10)


# ---------------------------------------------------------------------------
# special cases (spec invariants)
# ---------------------------------------------------------------------------

def test_exact_at_full_residual_rank():
    """rank(W_res) == r and X full column rank: Y = X W exactly (eps = 0)."""
    rng = _rng(50)
    c1, c2, k, r = 30, 40, 6, 4
    m = k + r
    U = synth.haar_columns(rng.standard_normal((c1, m)))
    V = synth.haar_columns(rng.standard_normal((c2, m)))
    W = (U * np.linspace(2.0, 0.5, m)) @ V.T
    X = _aniso_x(rng, 70, c1)
    bias = rng.standard_normal(c2)
    prep = _prep_lowrank(W, k, r)
    Y = O.forward(X, prep, bias, 1, 70, eps=0.0)
    np.testing.assert_allclose(Y, X @ W + bias, atol=1e-9)
    # the default small ridge leaves it exact to ~eps
    Y6 = O.forward(X, prep, bias, 1, 70, eps=1e-6)
    assert O.rel_fro(Y6 - bias, X @ W) < 1e-5


@pytest.mark.parametrize("kind", [O.KIND_MONARCH, O.KIND_BLAST])
def test_exact_when_r_is_full(kind):
    """r = min(c1, c2) with a full-rank generic residual reproduces X W."""
    rng = _rng(51)
    if kind == O.KIND_MONARCH:
        c, kw = 16, dict(mblk=4)
        W = rng.standard_normal((c, c))
        prep = O.prepare(W, kind, c, **kw)
    else:
        c, kw = 16, dict(nb=2, rb=3)
        W = rng.standard_normal((c, c))
        prep = O.prepare(W, kind, c, **kw)
    X = rng.standard_normal((40, c))
    Y = O.forward(X, prep, None, 1, 40, eps=0.0)
    np.testing.assert_allclose(Y, X @ W, atol=1e-9)


def test_zero_residual_gives_static_output():
    rng = _rng(52)
    c1, c2, k = 20, 24, 6
    U = synth.haar_columns(rng.standard_normal((c1, k)))
    V = synth.haar_columns(rng.standard_normal((c2, k)))
    W = (U * np.linspace(3, 1, k)) @ V.T                      # exactly rank k
    X = _aniso_x(rng, 30, c1)
    bias = rng.standard_normal(c2)
    prep = _prep_lowrank(W, k, 3)
    prep["W_res"] = np.zeros_like(W)
    prep["P"] = np.zeros_like(prep["P"])
    Y = O.forward(X, prep, bias, 1, 30, eps=1e-6)
    np.testing.assert_allclose(Y, X @ prep["W_hat"] + bias, atol=1e-12)


# ---------------------------------------------------------------------------
# structured matrices ([P2] App. B; [P5] structured-matrix section)
# ---------------------------------------------------------------------------

def test_lowrank_fit_closed_form_spectrum():
    """||W - W_hat||_F^2 = sum_{i>k} s_i^2 and the residual's top singular
    values are s_{k+1..k+r} when W = U diag(s) V^T (Eckart-Young)."""
    rng = _rng(60)
    c1, c2, k, r = 40, 64, 7, 5
    W, U, s, V = _power_law_w(rng, c1, c2)
    prep = _prep_lowrank(W, k, r)
    np.testing.assert_allclose(np.linalg.norm(prep["W_res"]) ** 2, np.sum(s[k:] ** 2), rtol=1e-10)
    np.testing.assert_allclose(prep["res_sv"], s[k:k + r], rtol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(prep["P"], axis=0), s[k:k + r], rtol=1e-10)
    # W_hat = X-independent best rank-k: equals U_k S_k V_k^T
    np.testing.assert_allclose(prep["W_hat"], (U[:, :k] * s[:k]) @ V[:, :k].T, atol=1e-12)


def test_monarch_factored_equals_dense():
    rng = _rng(61)
    m = 4
    f = {"B1": rng.standard_normal((m, m, m)), "B2": rng.standard_normal((m, m, m))}
    X = rng.standard_normal((7, m * m))
    np.testing.assert_allclose(O.monarch_apply(X, f), X @ O.monarch_dense(f), atol=1e-12)


def test_monarch_fit_recovers_exact_monarch_and_is_blockwise_optimal():
    rng = _rng(62)
    m = 5
    f = {"B1": rng.standard_normal((m, m, m)), "B2": rng.standard_normal((m, m, m))}
    W = O.monarch_dense(f)
    g = O.fit_monarch(W, m)
    np.testing.assert_allclose(O.monarch_dense(g), W, atol=1e-10)
    # generic W: the error is the sum of each block's tail singular values
    W2 = rng.standard_normal((m * m, m * m))
    Wh = O.monarch_dense(O.fit_monarch(W2, m))
    tail = sum(np.sum(np.linalg.svd(W2[a * m:(a + 1) * m, j * m:(j + 1) * m], compute_uv=False)[1:] ** 2)
               for a in range(m) for j in range(m))
    np.testing.assert_allclose(np.linalg.norm(W2 - Wh) ** 2, tail, rtol=1e-10)


def test_blast_factored_equals_dense():
    rng = _rng(63)
    nb, b1, b2, rb = 3, 4, 5, 2
    f = {"U": rng.standard_normal((nb, b1, rb)), "V": rng.standard_normal((nb, b2, rb)),
         "S": rng.standard_normal((nb, nb, rb, rb))}
    X = rng.standard_normal((6, nb * b1))
    np.testing.assert_allclose(O.blast_apply(X, f), X @ O.blast_dense(f), atol=1e-12)


def test_blast_fit_recovers_exact_blast_and_coupling_is_projection():
    rng = _rng(64)
    nb, b1, b2, rb = 3, 6, 8, 2
    f = {"U": np.stack([synth.haar_columns(rng.standard_normal((b1, rb))) for _ in range(nb)]),
         "V": np.stack([synth.haar_columns(rng.standard_normal((b2, rb))) for _ in range(nb)]),
         "S": rng.standard_normal((nb, nb, rb, rb))}
    W = O.blast_dense(f)
    g = O.fit_blast(W, nb, rb)
    np.testing.assert_allclose(O.blast_dense(g), W, atol=1e-10)
    W2 = rng.standard_normal((nb * b1, nb * b2))
    g2 = O.fit_blast(W2, nb, rb)
    E = W2 - O.blast_dense(g2)
    for i in range(nb):
        for j in range(nb):
            Eij = E[i * b1:(i + 1) * b1, j * b2:(j + 1) * b2]
            np.testing.assert_allclose(g2["U"][i].T @ Eij @ g2["V"][j], 0, atol=1e-12)


def test_blast_diagonal_fit_recovers_exact_diagonal_blast_and_is_entrywise_optimal():
    """Diagonal couplings.  W_ij = U_i diag(a_i b_j c) V_j^T with orthonormal
    bases and c decreasing: the Gram of block row i is U_i diag(a_i^2
    sum_j b_j^2 c^2) U_i^T, so its singular vectors are U_i's columns in the
    same order for every i (likewise V_j), and the fit recovers W.  (A
    generic diagonal-BLAST W is not identifiable by the one-pass bases: they
    are fixed only up to a rotation, which a diagonal coupling cannot
    absorb.)  On a generic W the couplings are diagonal, each entry is the
    projection u_p^T W_ij v_p (the residual has no component on the
    rank-one terms u_p v_p^T), equal to the full-coupling fit's diagonal,
    and the full-coupling fit is closer."""
    rng = _rng(66)
    nb, b1, b2, rb = 3, 6, 8, 2
    f = {"U": np.stack([synth.haar_columns(rng.standard_normal((b1, rb))) for _ in range(nb)]),
         "V": np.stack([synth.haar_columns(rng.standard_normal((b2, rb))) for _ in range(nb)]),
         "S": np.zeros((nb, nb, rb, rb))}
    a, b, c = rng.uniform(0.5, 2.0, nb), rng.uniform(0.5, 2.0, nb), np.array([3.0, 1.0])
    for i in range(nb):
        for j in range(nb):
            f["S"][i, j] = np.diag(a[i] * b[j] * c)
    W = O.blast_dense(f)
    g = O.fit_static(O.KIND_BLAST_DIAG, W, nb=nb, rb=rb)
    np.testing.assert_allclose(O.blast_dense(g), W, atol=1e-10)
    W2 = rng.standard_normal((nb * b1, nb * b2))
    d = O.fit_static(O.KIND_BLAST_DIAG, W2, nb=nb, rb=rb)
    full = O.fit_static(O.KIND_BLAST, W2, nb=nb, rb=rb)
    E = W2 - O.blast_dense(d)
    for i in range(nb):
        for j in range(nb):
            Sij = d["S"][i, j]
            np.testing.assert_array_equal(Sij, np.diag(np.diag(Sij)))
            Eij = E[i * b1:(i + 1) * b1, j * b2:(j + 1) * b2]
            np.testing.assert_allclose(np.diag(d["U"][i].T @ Eij @ d["V"][j]), 0, atol=1e-12)
            np.testing.assert_allclose(np.diag(Sij), np.diag(full["S"][i, j]), atol=1e-12)
    assert np.linalg.norm(W2 - O.blast_dense(full)) < np.linalg.norm(E)
    X = rng.standard_normal((5, nb * b1))
    np.testing.assert_allclose(O.static_apply(O.KIND_BLAST_DIAG, X, d), X @ O.blast_dense(d), atol=1e-12)


def test_blast_bases_are_top_singular_subspaces_of_block_rows_and_columns():
    """On a generic W, U_i spans the top-rb left singular subspace of the whole
    block row i and V_j the top-rb right singular subspace of the whole block
    column j: the projection errors equal the singular-value tails
    (Eckart-Young), which no other rb-dimensional basis attains."""
    rng = _rng(65)
    nb, b1, b2, rb = 3, 7, 6, 2
    W = rng.standard_normal((nb * b1, nb * b2))
    f = O.fit_blast(W, nb, rb)
    for i in range(nb):
        Wi = W[i * b1:(i + 1) * b1, :]
        Ui = f["U"][i]
        np.testing.assert_allclose(Ui.T @ Ui, np.eye(rb), atol=1e-12)
        tail = np.sum(np.linalg.svd(Wi, compute_uv=False)[rb:] ** 2)
        np.testing.assert_allclose(np.linalg.norm(Wi - Ui @ (Ui.T @ Wi)) ** 2, tail, rtol=1e-10)
    for j in range(nb):
        Wj = W[:, j * b2:(j + 1) * b2]
        Vj = f["V"][j]
        np.testing.assert_allclose(Vj.T @ Vj, np.eye(rb), atol=1e-12)
        tail = np.sum(np.linalg.svd(Wj, compute_uv=False)[rb:] ** 2)
        np.testing.assert_allclose(np.linalg.norm(Wj - (Wj @ Vj) @ Vj.T) ** 2, tail, rtol=1e-10)


# ---------------------------------------------------------------------------
# input-aware static start ([P2] App. B; [P5] structured-matrix section)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [O.INPUT_AWARE_DIAG, O.INPUT_AWARE_CHOL])
def test_input_aware_hand_worked(mode):
    """W = diag(2, 1), k = 1, calibration rows [1, 3] and [1, -3]: channel RMS
    (1, 3) and X^T X / n = diag(1, 9), so S = diag(1, 3) in both modes (up to
    the tiny ridge).  S W = diag(2, 3) keeps the 3 at (1, 1): W_hat =
    S^-1 diag(0, 3) = diag(0, 1), where the plain truncated SVD keeps
    diag(2, 0).  Derived by hand."""
    W = np.diag([2.0, 1.0])
    Xc = np.array([[1.0, 3.0], [1.0, -3.0]])
    prep = O.prepare(W, O.KIND_LOWRANK, 1, k=1, calib=(Xc, mode))
    np.testing.assert_allclose(prep["W_hat"], np.diag([0.0, 1.0]), atol=1e-6)
    np.testing.assert_allclose(O.prepare(W, O.KIND_LOWRANK, 1, k=1)["W_hat"], np.diag([2.0, 0.0]), atol=1e-12)


@pytest.mark.parametrize("mode", [O.INPUT_AWARE_DIAG, O.INPUT_AWARE_CHOL])
def test_input_aware_with_isotropic_calibration_is_the_plain_fit(mode):
    rng = _rng(90)
    W, *_ = _power_law_w(rng, 24, 30)
    Xc = synth.orthonormal_rows_input(rng, 48, 24, 2.5)       # X^T X / n = const I
    ia = O.prepare(W, O.KIND_LOWRANK, 3, k=5, calib=(Xc, mode))
    np.testing.assert_allclose(ia["W_hat"], _prep_lowrank(W, 5, 3)["W_hat"], atol=1e-9)


def test_input_aware_cholesky_fit_is_optimal_in_the_calibration_norm():
    """||X_cal (W - W_hat)||_F^2 / n equals the singular-value tail of C^T W
    (Eckart-Young in the weighted norm) and is below the plain fit's."""
    rng = _rng(91)
    W, *_ = _power_law_w(rng, 20, 28)
    Xc = _aniso_x(rng, 200, 20)
    k = 6
    ia = O.prepare(W, O.KIND_LOWRANK, 3, k=k, calib=(Xc, O.INPUT_AWARE_CHOL))
    n, c1 = Xc.shape
    K = Xc.T @ Xc / n
    C = np.linalg.cholesky(K + O.CALIB_RIDGE * np.trace(K) / c1 * np.eye(c1))
    tail = np.sum(np.linalg.svd(C.T @ W, compute_uv=False)[k:] ** 2)
    E = W - ia["W_hat"]
    np.testing.assert_allclose(np.linalg.norm(C.T @ E) ** 2, tail, rtol=1e-9)
    plain = W - _prep_lowrank(W, k, 3)["W_hat"]
    assert np.linalg.norm(Xc @ E) < np.linalg.norm(Xc @ plain)
    assert np.linalg.matrix_rank(ia["W_hat"], tol=1e-9) == k


def test_input_aware_diagonal_fit_is_optimal_in_the_scaled_norm():
    rng = _rng(92)
    W, *_ = _power_law_w(rng, 20, 28)
    Xc = _aniso_x(rng, 100, 20)
    k = 4
    ia = O.prepare(W, O.KIND_LOWRANK, 3, k=k, calib=(Xc, O.INPUT_AWARE_DIAG))
    s = np.sqrt(np.mean(Xc ** 2, axis=0))
    tail = np.sum(np.linalg.svd(s[:, None] * W, compute_uv=False)[k:] ** 2)
    np.testing.assert_allclose(np.linalg.norm(s[:, None] * (W - ia["W_hat"])) ** 2, tail, rtol=1e-9)
    # the residual split stays exact: W_hat + W_res = W, P = W_res R0^T
    np.testing.assert_allclose(ia["W_hat"] + ia["W_res"], W, atol=1e-12)
    np.testing.assert_allclose(ia["P"], ia["W_res"] @ ia["R0"].T, atol=1e-12)


# ---------------------------------------------------------------------------
# invariances (readings: per-segment solve, relative ridge, R0 rotation)
# ---------------------------------------------------------------------------

def _setup(seed=70, kind=O.KIND_LOWRANK):
    rng = _rng(seed)
    if kind == O.KIND_LOWRANK:
        W, *_ = _power_law_w(rng, 32, 40)
        prep = _prep_lowrank(W, 8, 5)
        c1 = 32
    elif kind == O.KIND_MONARCH:
        W, *_ = _power_law_w(rng, 16, 16)
        prep = O.prepare(W, kind, 5, mblk=4)
        c1 = 16
    else:
        W, *_ = _power_law_w(rng, 16, 24)
        prep = O.prepare(W, kind, 5, nb=2, rb=3)
        c1 = 16
    X = _aniso_x(rng, 3 * 20, c1)
    bias = rng.standard_normal(W.shape[1])
    return rng, W, prep, X, bias


@pytest.mark.parametrize("kind", [O.KIND_LOWRANK, O.KIND_MONARCH, O.KIND_BLAST])
def test_homogeneity(kind):
    _, _, prep, X, bias = _setup(kind=kind)
    Y1 = O.forward(X, prep, bias, 3, 20)
    Y2 = O.forward(2.5 * X, prep, bias, 3, 20)
    np.testing.assert_allclose(Y2 - bias, 2.5 * (Y1 - bias), rtol=1e-9, atol=1e-12)


def test_row_permutation_equivariance_and_segment_independence():
    rng, _, prep, X, bias = _setup()
    Y = O.forward(X, prep, bias, 3, 20)
    perm = rng.permutation(20)
    Xp = X.copy()
    Xp[20:40] = X[20:40][perm]
    Yp = O.forward(Xp, prep, bias, 3, 20)
    np.testing.assert_allclose(Yp[20:40], Y[20:40][perm], atol=1e-12)
    np.testing.assert_allclose(Yp[:20], Y[:20], atol=0)
    for b in range(3):
        Yb = O.forward(X[b * 20:(b + 1) * 20], prep, bias, 1, 20)
        np.testing.assert_allclose(Yb, Y[b * 20:(b + 1) * 20], atol=1e-13)


def test_ragged_segments_are_independent_forwards():
    """Segments given by row offsets: each is its own ALS solve, so the
    ragged forward is the concatenation of one-segment forwards, and uniform
    offsets reproduce the B x s forward bit for bit."""
    rng, _, prep, X, bias = _setup()
    off = [0, 1, 9, 23, 60]                       # lengths 1, 8, 14, 37 (one shorter than r = 5)
    Y = O.forward(X, prep, bias, 0, 0, offsets=off)
    for lo, hi in zip(off[:-1], off[1:]):
        np.testing.assert_array_equal(Y[lo:hi], O.forward(X[lo:hi], prep, bias, 1, hi - lo))
    np.testing.assert_array_equal(O.forward(X, prep, bias, 0, 0, offsets=[0, 20, 40, 60]),
                                  O.forward(X, prep, bias, 3, 20))


def test_ragged_segments_are_independent_at_more_iterations():
    """The same at t = 1.5 and t = 2: every ALS half-step of a segment uses
    that segment's rows only, so moving a boundary changes only the two
    segments it separates."""
    rng, _, prep, X, bias = _setup()
    off = [0, 9, 23, 60]
    for t in (1.5, 2.0):
        Y = O.forward(X, prep, bias, 0, 0, t=t, offsets=off)
        for lo, hi in zip(off[:-1], off[1:]):
            np.testing.assert_array_equal(Y[lo:hi], O.forward(X[lo:hi], prep, bias, 1, hi - lo, t=t))
        Y2 = O.forward(X, prep, bias, 0, 0, t=t, offsets=[0, 9, 30, 60])
        np.testing.assert_array_equal(Y2[:9], Y[:9])
        assert not np.allclose(Y2[9:23], Y[9:23])


def test_rotation_of_initial_right_factor_changes_nothing():
    rng, _, prep, X, bias = _setup()
    Q = synth.haar_columns(rng.standard_normal((5, 5)))
    rot = dict(prep)
    rot["R0"] = Q @ prep["R0"]
    rot["P"] = prep["P"] @ Q.T
    np.testing.assert_allclose(O.forward(X, rot, bias, 3, 20), O.forward(X, prep, bias, 3, 20),
                               atol=1e-11)


# ---------------------------------------------------------------------------
# r x r solvers ([P2] 2.4)
# ---------------------------------------------------------------------------

def test_newton_schulz_converges_to_inverse():
    rng = _rng(80)
    A = np.diag([4.0, 2.0, 0.5])
    Xi, it, ok = O.newton_schulz_inverse(A, tol=1e-12)
    assert ok
    np.testing.assert_allclose(Xi, np.diag([0.25, 0.5, 2.0]), rtol=1e-11)
    L = rng.standard_normal((200, 24)) * np.linspace(3, 0.3, 24)
    G = L.T @ L
    Gi, it, ok = O.newton_schulz_inverse(G, tol=1e-10, maxit=60)
    assert ok
    np.testing.assert_allclose(G @ Gi, np.eye(24), atol=1e-9)


def test_cholesky_textbook_matches_definition():
    rng = _rng(81)
    L = rng.standard_normal((50, 9))
    G = L.T @ L + 0.1 * np.eye(9)
    C = O.cholesky_lower(G)
    np.testing.assert_allclose(C @ C.T, G, atol=1e-12)
    assert np.allclose(C, np.tril(C))
    np.testing.assert_allclose(C, sla.cholesky(G, lower=True), atol=1e-12)


@pytest.mark.parametrize("sin2,singular", [(2.0 ** -15, False), (2.0 ** -17, True), (0.0, True)])
def test_unridged_solve_rank_test_on_two_columns(sin2, singular):
    """eps = 0: two unit columns at an angle theta give K = [[1, c], [c, 1]]
    with Cholesky pivots 1 and 1 - c^2 = sin^2 theta; the system counts as
    singular exactly when sin^2 theta <= 2^-16, and then the solve gives 0."""
    c = np.sqrt(1.0 - sin2)
    K = np.array([[1.0, c], [c, 1.0]])
    assert O.gram_is_singular(K) == singular
    rhs = np.array([[1.0, 2.0], [3.0, -1.0]])
    Z = O.spd_solve(K, rhs, 0.0)
    if singular:
        assert not np.any(Z)
    else:
        np.testing.assert_allclose(K @ Z, rhs, atol=1e-9 / sin2)


def test_unridged_forward_with_fewer_tokens_than_rank_falls_back_to_static():
    """s < r at eps = 0: L_b has rank s < r, G_b is singular, R_b = 0 and the
    segment's output is exactly X_b W_hat + bias; with a ridge it is not."""
    rng = _rng(83)
    W, *_ = _power_law_w(rng, 24, 32)
    prep = _prep_lowrank(W, 4, 6)
    X = _aniso_x(rng, 2 * 4, 24)                                  # 2 segments of 4 tokens, r = 6
    bias = rng.standard_normal(32)
    Y0 = O.forward(X, prep, bias, 2, 4, eps=0.0)
    np.testing.assert_allclose(Y0, X @ prep["W_hat"] + bias, atol=1e-12)
    Y6 = O.forward(X, prep, bias, 2, 4, eps=1e-6)
    assert O.rel_fro(Y6, X @ prep["W_hat"] + bias) > 1e-3


def test_spd_solve_zero_trace_guard():
    G = np.zeros((3, 3))
    H = np.ones((3, 4))
    assert not np.any(O.spd_solve(G, H, 1e-6))


# ---------------------------------------------------------------------------
# generator facts the tests rely on
# ---------------------------------------------------------------------------

def test_generator_spectrum_and_rounding():
    w = synth.scaled(synth.WORKLOADS["vitb_fc1"], B=2, s=8, c1=64, c2=96, k=8, r=8)
    inp = synth.make_inputs(w)
    np.testing.assert_allclose(np.linalg.svd(inp.W_exact, compute_uv=False), inp.spectrum, rtol=1e-10)
    assert np.array_equal(synth.round_bf16(inp.X), inp.X)
    assert np.array_equal(synth.round_bf16(inp.W), inp.W)
    # RNE ties: 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7 -> even (1)
    assert synth.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert synth.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
