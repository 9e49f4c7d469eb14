"""DyRA oracle: a plain, slow, float64 CPU statement of the DyRA layer forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product library never calls it,
and it shares no code with the HIP path (it imports numpy/scipy only).

Source pages (cited by title and section; the paper is arXiv 2610.02882,
"DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
DNNs"):
  [P2]  the paperlayer.ai section-by-section summary of the paper
        (sections 2.2, 2.3, 2.4, App. B "Background on Structured Matrices",
        App. C "Proof of Proposition 1", E.3, E.4).
  [P5]  the nanless.github.io digest blog post on DyRA (Chinese), sections
        "how the static branch and the residual are split" (equations
        W = W_hat + W_res and XW = X W_hat + X W_res), "what the low-rank
        objective of the residual product is" (min over L, R of
        ||X W_res - L R||_F^2 and the ALS ordering), "one-iteration form and
        extra cost" (equation XW ~ X W_hat + ALS_1(X W_res) = X W_hat + L1 R1),
        "overall DyRA flow", "how the existing structured-matrix methods
        differ", "offline preparation and online computation without
        training", "first reproduction step" (small ridge).

Readings taken where the pages leave a step open:
  * one input = one segment of s consecutive rows; B segments are solved
    independently.
  * R0 = top-r right singular vectors of W_res (orthonormal rows), so the
    first left step is L = X P with P = W_res R0^T.
  * ridge: lambda = eps * trace(G) / r added to G = L^T L; trace(G) == 0
    gives R = 0.  eps == 0 (no ridge) solves the normal equations by
    Cholesky when G is numerically nonsingular (every pivot above 2^-16 of
    its diagonal) and otherwise drops the correction (R = 0).
  * Monarch: W_hat = blockdiag(B1_a) . Pi . blockdiag(B2_j), Pi the
    reshape(m, m)-transpose permutation, each (a, j) block of W fitted by
    its rank-1 truncated SVD.
  * BLAST: block row bases U_i = top-rb left singular vectors of block row
    i, block column bases V_j = top-rb right singular vectors of block
    column j, coupling S_ij = U_i^T W_ij V_j (general rb x rb).
  * low-rank factors split sqrt(sigma) to each side.

Parity pins (tests/test_oracle_pins.py): hand-derived worked examples,
Proposition 1 closed form, brute-force least squares, orthogonality,
never-worse-than-static, Eckart-Young bound, exactness at full residual
rank, W_res = 0, structured forward = dense product, exact structured fits,
closed-form spectra, invariances, solver identities.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg as sla

KIND_LOWRANK = 0
KIND_MONARCH = 1
KIND_BLAST = 2
KIND_BLAST_DIAG = 3     # BLAST with diagonal couplings S_ij = diag(s_ij)


# ---------------------------------------------------------------------------
# Static structured approximations  ([P2] App. B; [P5] "how the existing
# structured-matrix methods differ")
# ---------------------------------------------------------------------------

def fit_lowrank(W: np.ndarray, k: int) -> dict:
    """Truncated SVD: keep the top-k singular triplets of W (best rank-k in
    Frobenius norm), split as U_f = U_k sqrt(S_k), V_f = sqrt(S_k) V_k^T."""
    U, s, Vt = np.linalg.svd(W, full_matrices=False)
    rs = np.sqrt(s[:k])
    return {"U": U[:, :k] * rs, "V": rs[:, None] * Vt[:k], "sv": s}


def lowrank_dense(f: dict) -> np.ndarray:
    return f["U"] @ f["V"]


def lowrank_apply(X: np.ndarray, f: dict) -> np.ndarray:
    """Static branch as two thin products X U_f, then (X U_f) V_f."""
    return (X @ f["U"]) @ f["V"]


def fit_monarch(W: np.ndarray, m: int) -> dict:
    """Monarch fit by a rank-1 truncated SVD of every m x m block of W.

    W_hat[(a,i),(j,l)] = B1[a][i, j] * B2[j][a, l]: block (a, j) of W_hat is
    the outer product of column j of B1[a] and row a of B2[j].
    """
    c = m * m
    assert W.shape == (c, c)
    B1 = np.zeros((m, m, m))
    B2 = np.zeros((m, m, m))
    for a in range(m):
        for j in range(m):
            blk = W[a * m:(a + 1) * m, j * m:(j + 1) * m]
            U, s, Vt = np.linalg.svd(blk)
            B1[a][:, j] = np.sqrt(s[0]) * U[:, 0]
            B2[j][a, :] = np.sqrt(s[0]) * Vt[0]
    return {"B1": B1, "B2": B2}


def monarch_permutation(m: int) -> np.ndarray:
    """Pi with (x Pi)[j*m + a] = x[a*m + j] (reshape to m x m, transpose)."""
    c = m * m
    Pi = np.zeros((c, c))
    for a in range(m):
        for j in range(m):
            Pi[a * m + j, j * m + a] = 1.0
    return Pi


def monarch_dense(f: dict) -> np.ndarray:
    """W_hat = blockdiag(B1) . Pi . blockdiag(B2) as explicit dense matrices."""
    B1, B2 = f["B1"], f["B2"]
    m = B1.shape[0]
    return sla.block_diag(*B1) @ monarch_permutation(m) @ sla.block_diag(*B2)


def monarch_apply(X: np.ndarray, f: dict) -> np.ndarray:
    """Factored Monarch product: per-block stage 1, permutation, stage 2."""
    B1, B2 = f["B1"], f["B2"]
    m = B1.shape[0]
    n = X.shape[0]
    u = np.einsum("tai,aij->taj", X.reshape(n, m, m), B1)     # stage 1, block a
    v = u.transpose(0, 2, 1)                                    # Pi: v[t, j, a]
    y = np.einsum("tja,jal->tjl", v, B2)                        # stage 2, block j
    return y.reshape(n, m * m)


def fit_blast(W: np.ndarray, nb: int, rb: int, diagonal: bool = False) -> dict:
    """BLAST fit on an nb x nb block grid with shared rank-rb bases.

    U[i] (c1/nb x rb): top-rb left singular vectors of block row i.
    V[j] (c2/nb x rb): top-rb right singular vectors of block column j.
    S[i, j] = U[i]^T W_ij V[j]: the least-squares coupling for these bases;
    with diagonal couplings only its diagonal is kept, which is the
    least-squares diagonal coupling for orthonormal bases (entry p fits the
    rank-one term u_p v_p^T, and those terms are orthonormal).
    """
    c1, c2 = W.shape
    b1, b2 = c1 // nb, c2 // nb
    U = np.zeros((nb, b1, rb))
    V = np.zeros((nb, b2, rb))
    S = np.zeros((nb, nb, rb, rb))
    for i in range(nb):
        Ui, _, _ = np.linalg.svd(W[i * b1:(i + 1) * b1, :], full_matrices=False)
        U[i] = Ui[:, :rb]
    for j in range(nb):
        _, _, Vt = np.linalg.svd(W[:, j * b2:(j + 1) * b2], full_matrices=False)
        V[j] = Vt[:rb].T
    for i in range(nb):
        for j in range(nb):
            S[i, j] = U[i].T @ W[i * b1:(i + 1) * b1, j * b2:(j + 1) * b2] @ V[j]
            if diagonal:
                S[i, j] = np.diag(np.diag(S[i, j]))
    return {"U": U, "V": V, "S": S}


def blast_dense(f: dict) -> np.ndarray:
    U, V, S = f["U"], f["V"], f["S"]
    nb = U.shape[0]
    rows = []
    for i in range(nb):
        rows.append(np.hstack([U[i] @ S[i, j] @ V[j].T for j in range(nb)]))
    return np.vstack(rows)


def blast_apply(X: np.ndarray, f: dict) -> np.ndarray:
    """Factored BLAST product: z_i = x_i U_i, w_j = sum_i z_i S_ij, y_j = w_j V_j^T."""
    U, V, S = f["U"], f["V"], f["S"]
    nb, b1, _ = U.shape
    z = [X[:, i * b1:(i + 1) * b1] @ U[i] for i in range(nb)]
    out = []
    for j in range(nb):
        w = sum(z[i] @ S[i, j] for i in range(nb))
        out.append(w @ V[j].T)
    return np.hstack(out)


# ---------------------------------------------------------------------------
# Input-aware static start ([P2] App. B "Background on Structured Matrices";
# [P5] "how the existing structured-matrix methods differ": a transform S
# built from calibration activations, the weight written through S and its
# inverse, and a truncated SVD of the transformed weight).  With Y = X W the
# transform acts on the input side: W_hat = S^-1 SVD_k(S W), which for
# S^T S = X_cal^T X_cal / n is the rank-k W_hat closest to W in the
# calibration output norm ||X_cal (W - W_hat)||_F.
# ---------------------------------------------------------------------------

INPUT_AWARE_DIAG = 1      # S = diag(channel RMS over the calibration rows)
INPUT_AWARE_CHOL = 2      # S = C^T, C C^T = X_cal^T X_cal / n + delta I
CALIB_RIDGE = 1e-6        # delta = CALIB_RIDGE * trace(X_cal^T X_cal / n) / c1
CALIB_FLOOR = 1e-6        # a channel RMS below CALIB_FLOOR * the largest is raised to it


def input_transform(X_cal: np.ndarray, mode: int) -> np.ndarray:
    """The c1 x c1 transform S of an input-aware fit."""
    n, c1 = X_cal.shape
    if mode == INPUT_AWARE_DIAG:
        rms = np.sqrt(np.mean(X_cal * X_cal, axis=0))
        return np.diag(np.maximum(rms, CALIB_FLOOR * rms.max()))
    if mode == INPUT_AWARE_CHOL:
        K = X_cal.T @ X_cal / n
        K = K + CALIB_RIDGE * np.trace(K) / c1 * np.eye(c1)
        return cholesky_lower(K).T
    raise ValueError(mode)


def fit_lowrank_input_aware(W: np.ndarray, k: int, S: np.ndarray) -> dict:
    """W_hat = S^-1 SVD_k(S W), split as U_f = S^-1 U_k sqrt(s_k),
    V_f = sqrt(s_k) V_k^T (the sqrt(sigma) split of the plain fit)."""
    U, s, Vt = np.linalg.svd(S @ W, full_matrices=False)
    rs = np.sqrt(s[:k])
    return {"U": np.linalg.solve(S, U[:, :k] * rs), "V": rs[:, None] * Vt[:k], "sv": s}


def static_dense(kind: int, f: dict) -> np.ndarray:
    return {KIND_LOWRANK: lowrank_dense, KIND_MONARCH: monarch_dense,
            KIND_BLAST: blast_dense, KIND_BLAST_DIAG: blast_dense}[kind](f)


def static_apply(kind: int, X: np.ndarray, f: dict) -> np.ndarray:
    return {KIND_LOWRANK: lowrank_apply, KIND_MONARCH: monarch_apply,
            KIND_BLAST: blast_apply, KIND_BLAST_DIAG: blast_apply}[kind](X, f)


def fit_static(kind: int, W: np.ndarray, k=0, mblk=0, nb=0, rb=0) -> dict:
    if kind == KIND_LOWRANK:
        return fit_lowrank(W, k)
    if kind == KIND_MONARCH:
        return fit_monarch(W, mblk)
    if kind in (KIND_BLAST, KIND_BLAST_DIAG):
        return fit_blast(W, nb, rb, diagonal=kind == KIND_BLAST_DIAG)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# Offline preparation  ([P5] "overall DyRA flow" and "offline preparation and
# online computation without training"; [P2] App. A names the two stages)
# ---------------------------------------------------------------------------

def residual_init(W_res: np.ndarray, r: int):
    """Fixed initial right factor R0 (r x c2): the top-r right singular
    vectors of W_res; thin projection P = W_res R0^T (c1 x r)."""
    _, rho, Vt = np.linalg.svd(W_res, full_matrices=False)
    R0 = Vt[:r].copy()
    return R0, W_res @ R0.T, rho[:r]


def prepare(W: np.ndarray, kind: int, r: int, k=0, mblk=0, nb=0, rb=0, calib=None) -> dict:
    """W = W_hat + W_res; R0, P from the residual  ([P5] split equation).
    calib = (X_cal, mode): the input-aware static start (low-rank only)."""
    if calib is not None:
        if kind != KIND_LOWRANK:
            raise ValueError("the input-aware fit is a truncated SVD: low-rank only")
        f = fit_lowrank_input_aware(W, k, input_transform(calib[0], calib[1]))
    else:
        f = fit_static(kind, W, k=k, mblk=mblk, nb=nb, rb=rb)
    W_hat = static_dense(kind, f)
    W_res = W - W_hat
    R0, P, rho = residual_init(W_res, r)
    return {"kind": kind, "static": f, "W_hat": W_hat, "W_res": W_res,
            "R0": R0, "P": P, "res_sv": rho, "r": r}


# ---------------------------------------------------------------------------
# ALS half-steps  ([P5] "what the low-rank objective of the residual product
# is": min over L (n x r), R (r x c2) of ||X W_res - L R||_F^2; [P2] 2.2)
# ---------------------------------------------------------------------------

def ridge(K: np.ndarray, eps: float) -> float:
    """lambda = eps * trace(K) / r: the small ridge of [P2] 2.2, scaled so the
    output stays homogeneous of degree one in X."""
    r = K.shape[0]
    return eps * np.trace(K) / r


# eps == 0 only: a Cholesky pivot d_j (the squared distance of column j of L
# from the span of the earlier columns) at or below SINGULAR_PIVOT_REL times
# the diagonal K_jj (the squared length of column j) marks K as singular.
SINGULAR_PIVOT_REL = 2.0 ** -16


def gram_is_singular(K: np.ndarray) -> bool:
    """Numerical rank test of an unridged Gram matrix K = L^T L: a Cholesky
    pivot d_j <= SINGULAR_PIVOT_REL * K_jj (sin^2 of the angle between column
    j and the earlier columns), or a non-positive pivot."""
    r = K.shape[0]
    C = np.zeros_like(K)
    for j in range(r):
        d = K[j, j] - C[j, :j] @ C[j, :j]
        if not d > SINGULAR_PIVOT_REL * K[j, j]:
            return True
        C[j, j] = np.sqrt(d)
        C[j + 1:, j] = (K[j + 1:, j] - C[j + 1:, :j] @ C[j, :j]) / C[j, j]
    return False


def spd_solve(K: np.ndarray, rhs: np.ndarray, eps: float) -> np.ndarray:
    """Solve (K + lambda I) Z = rhs for symmetric PSD K.

    eps > 0: Cholesky solve ([P2] 2.4 names Cholesky for small r).
    eps == 0 (no ridge; the pages always add one): the Cholesky solve of the
    normal equations when K is numerically nonsingular (gram_is_singular),
    else Z = 0: the correction is dropped rather than fitted to a singular
    system, so the output falls back to the static branch.
    trace(K) == 0: Z = 0.
    """
    if not np.any(K):
        return np.zeros_like(rhs)
    if eps > 0:
        lam = ridge(K, eps)
        return sla.cho_solve(sla.cho_factor(K + lam * np.eye(K.shape[0]), lower=True), rhs)
    if gram_is_singular(K):
        return np.zeros_like(rhs)
    return sla.cho_solve(sla.cho_factor(K, lower=True), rhs)


def right_step(X: np.ndarray, W_res: np.ndarray, L: np.ndarray, eps: float) -> np.ndarray:
    """Fix L, solve for R: R = (L^T L + lambda I)^-1 (L^T X) W_res.

    The input is projected to L's r dimensions first (L^T X is r x c1), then
    multiplied by W_res, so the n x c2 product X W_res is never formed.
    """
    G = L.T @ L
    M = L.T @ X
    H = M @ W_res
    return spd_solve(G, H, eps)


def left_step(X: np.ndarray, W_res: np.ndarray, R: np.ndarray, eps: float) -> np.ndarray:
    """Fix R, solve for L: L = X (W_res R^T) (R R^T + lambda I)^-1.

    The residual is projected to R's r dimensions first (W_res R^T is
    c1 x r), then X multiplies that thin matrix.
    """
    Q = W_res @ R.T
    K = R @ R.T
    return X @ spd_solve(K, Q.T, eps).T


def als(X: np.ndarray, W_res: np.ndarray, R0: np.ndarray, t: float, eps: float,
        P: np.ndarray | None = None):
    """ALS on X W_res started from R0.  t = 1: one L update then one R update
    (the default of [P2] 3.3); t = 1.5: L, R, L; t = 2: L, R, L, R.

    The first L update uses the precomputed thin matrix P = W_res R0^T when
    given (valid since R0 has orthonormal rows)."""
    half_steps = int(round(2 * t))
    L = X @ P if P is not None else left_step(X, W_res, R0, eps)
    R = R0
    for h in range(1, half_steps):
        if h % 2 == 1:
            R = right_step(X, W_res, L, eps)
        else:
            L = left_step(X, W_res, R, eps)
    return L, R


# ---------------------------------------------------------------------------
# Layer forward  ([P5] "one-iteration form": XW ~ X W_hat + L1 R1;
# [P2] 2.4: bias is merged with the base projection and the correction)
# ---------------------------------------------------------------------------

def segment_rows(B: int, s: int, offsets=None) -> list:
    """Row ranges of the segments: B runs of s rows, or rows offsets[b] ..
    offsets[b + 1] - 1 (ragged segments, e.g. prompts of mixed length)."""
    if offsets is None:
        return [(b * s, (b + 1) * s) for b in range(B)]
    return [(int(offsets[b]), int(offsets[b + 1])) for b in range(len(offsets) - 1)]


def forward(X: np.ndarray, prep: dict, bias: np.ndarray | None, B: int, s: int,
            eps: float = 1e-6, t: float = 1.0, offsets=None) -> np.ndarray:
    """Y = X W_hat + L R + bias, with (L, R) from ALS on each segment
    (B segments of s rows, or the ragged segments of `offsets`)."""
    n, c1 = X.shape
    rows = segment_rows(B, s, offsets)
    assert rows[0][0] == 0 and rows[-1][1] == n
    kind, f, W_res, R0, P = prep["kind"], prep["static"], prep["W_res"], prep["R0"], prep["P"]
    Y = np.empty((n, W_res.shape[1]))
    for lo, hi in rows:
        Xb = X[lo:hi]
        base = static_apply(kind, Xb, f)
        L, R = als(Xb, W_res, R0, t, eps, P=P if t >= 1 else None)
        Y[lo:hi] = base + L @ R
    if bias is not None:
        Y += bias[None, :]
    return Y


def forward_segment_factors(Xb: np.ndarray, W_res: np.ndarray, P: np.ndarray, eps: float):
    """The one-step factors of a single segment: L, G, lambda, M, R."""
    L = Xb @ P
    G = L.T @ L
    lam = ridge(G, eps)
    M = L.T @ Xb
    R = spd_solve(G, M @ W_res, eps)
    return {"L": L, "G": G, "lam": lam, "M": M, "R": R}


# ---------------------------------------------------------------------------
# r x r SPD solvers  ([P2] 2.4: Cholesky for small r, Newton-Schulz for large r)
# ---------------------------------------------------------------------------

def newton_schulz_inverse(A: np.ndarray, tol: float = 1e-6, maxit: int = 40):
    """Newton-Schulz iteration for A^-1 (A SPD):
    X0 = I / ||A||_F,  X_{k+1} = X_k (2 I - A X_k), until ||I - A X_k||_F <= tol.
    Returns (X, iterations, converged)."""
    r = A.shape[0]
    I = np.eye(r)
    Xk = I / np.linalg.norm(A)
    for it in range(1, maxit + 1):
        Xk = Xk @ (2.0 * I - A @ Xk)
        if np.linalg.norm(I - A @ Xk) <= tol:
            return Xk, it, True
    return Xk, maxit, False


def cholesky_lower(A: np.ndarray) -> np.ndarray:
    """Textbook column Cholesky A = C C^T (C lower), no library call."""
    r = A.shape[0]
    C = np.zeros_like(A)
    for j in range(r):
        d = A[j, j] - C[j, :j] @ C[j, :j]
        C[j, j] = np.sqrt(d)
        for i in range(j + 1, r):
            C[i, j] = (A[i, j] - C[i, :j] @ C[j, :j]) / C[j, j]
    return C


# ---------------------------------------------------------------------------
# error metrics
# ---------------------------------------------------------------------------

def rel_fro(A: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(A - ref) / (d if d > 0 else 1.0))
