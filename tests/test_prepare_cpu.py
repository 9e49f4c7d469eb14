"""The library's host preparation (C++ float64) against the oracle's, and the
device-plan packing layout (CPU only).  Comparisons are invariant to the sign
and rotation freedom of singular vectors: dense W_hat, the residual, the
projector R0^T R0, R0 R0^T = I, P = W_res R0^T and the singular values."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O


def _w(seed, c1, c2):
    rng = np.random.default_rng(seed)
    m = min(c1, c2)
    U = synth.haar_columns(rng.standard_normal((c1, m)))
    V = synth.haar_columns(rng.standard_normal((c2, m)))
    return (U * np.arange(1, m + 1) ** -0.5) @ V.T


def _check_common(f, o, W, r):
    # residual, singular values, R0 orthonormal, same top-r right subspace, P
    np.testing.assert_allclose(f["Wres"], o["W_res"], atol=1e-10)
    np.testing.assert_allclose(f["res_sv"], o["res_sv"], rtol=1e-9)
    np.testing.assert_allclose(f["R0"] @ f["R0"].T, np.eye(r), atol=1e-10)
    np.testing.assert_allclose(f["R0"].T @ f["R0"], o["R0"].T @ o["R0"], atol=1e-8)
    np.testing.assert_allclose(f["P"], f["Wres"] @ f["R0"].T, atol=1e-10)
    np.testing.assert_allclose(f["P"] @ f["R0"], o["P"] @ o["R0"], atol=1e-8)


@pytest.mark.parametrize("c1,c2,k,r", [(64, 96, 16, 8), (96, 64, 24, 16), (128, 128, 32, 32)])
def test_prepare_lowrank_matches_oracle(c1, c2, k, r):
    W = _w(c1 + c2, c1, c2)
    spec = D.make_spec(synth.KIND_LOWRANK, c1, c2, r, k=k)
    f = D.prepare(W, spec, nthreads=4)
    o = O.prepare(W, O.KIND_LOWRANK, r, k=k)
    np.testing.assert_allclose(f["U"] @ f["V"], o["W_hat"], atol=1e-10)
    # sqrt(sigma) split: column norms of U_f equal row norms of V_f
    np.testing.assert_allclose(np.linalg.norm(f["U"], axis=0), np.linalg.norm(f["V"], axis=1), rtol=1e-9)
    _check_common(f, o, W, r)


def test_prepare_monarch_matches_oracle():
    m, r = 8, 16
    W = _w(5, m * m, m * m)
    spec = D.make_spec(synth.KIND_MONARCH, m * m, m * m, r, mblk=m)
    f = D.prepare(W, spec, nthreads=4)
    o = O.prepare(W, O.KIND_MONARCH, r, mblk=m)
    np.testing.assert_allclose(O.monarch_dense({"B1": f["B1"], "B2": f["B2"]}), o["W_hat"], atol=1e-10)
    _check_common(f, o, W, r)


def test_prepare_blast_matches_oracle():
    nb, rb, r = 4, 8, 16
    W = _w(6, 64, 96)
    spec = D.make_spec(synth.KIND_BLAST, 64, 96, r, nb=nb, rb=rb)
    f = D.prepare(W, spec, nthreads=4)
    o = O.prepare(W, O.KIND_BLAST, r, nb=nb, rb=rb)
    np.testing.assert_allclose(O.blast_dense({"U": f["Ub"], "V": f["Vb"], "S": f["S"]}), o["W_hat"],
                               atol=1e-10)
    _check_common(f, o, W, r)


def test_prepare_exact_lowrank_residual_zero():
    """A weight of exact rank k: W_res = 0, R0 still orthonormal, P = 0."""
    rng = np.random.default_rng(7)
    U = synth.haar_columns(rng.standard_normal((48, 8)))
    V = synth.haar_columns(rng.standard_normal((64, 8)))
    W = (U * np.linspace(2, 1, 8)) @ V.T
    spec = D.make_spec(synth.KIND_LOWRANK, 48, 64, 8, k=8)
    f = D.prepare(W, spec, nthreads=2)
    assert np.abs(f["Wres"]).max() < 1e-12
    assert np.abs(f["P"]).max() < 1e-12
    np.testing.assert_allclose(f["R0"] @ f["R0"].T, np.eye(8), atol=1e-10)


def test_prepare_vitb_shape_closed_form():
    """At the ViT-B fc1 shape: residual spectrum = s_{k+1..k+r} of the
    generator's power law (Eckart-Young), checked against the closed form."""
    w = synth.WORKLOADS["vitb_fc1"]
    inp = synth.make_inputs(synth.scaled(w, B=1, s=8))
    spec = D.spec_of(w)
    f = D.prepare(inp.W_exact, spec)
    np.testing.assert_allclose(f["res_sv"], inp.spectrum[w.k:w.k + w.r], rtol=1e-8)
    np.testing.assert_allclose(np.linalg.norm(f["Wres"]) ** 2, np.sum(inp.spectrum[w.k:] ** 2), rtol=1e-9)


def _bf16(a):
    return synth.round_bf16(a)


def test_plan_pack_lowrank_layout():
    c1, c2, k, r = 64, 96, 16, 8
    spec = D.make_spec(synth.KIND_LOWRANK, c1, c2, r, k=k)
    f = D.prepare(_w(1, c1, c2), spec)
    for dtype in (synth.DT_F32, synth.DT_BF16):
        buf = D.plan_pack(spec, f, dtype)
        if dtype == synth.DT_BF16:
            vals = synth.bf16_to_f64(buf.view(np.uint16))
            rnd = _bf16
            esz = 2
        else:
            vals = buf.view(np.float32).astype(np.float64)
            rnd = synth.round_f32
            esz = 4
        off = 0
        UPt = vals[off:off + (k + r) * c1].reshape(k + r, c1)
        np.testing.assert_array_equal(UPt[:k], rnd(f["U"].T))
        np.testing.assert_array_equal(UPt[k:], rnd(f["P"].T))
        off = ((k + r) * c1 * esz + 255) // 256 * 256 // esz
        Vt = vals[off:off + c2 * k].reshape(c2, k)
        np.testing.assert_array_equal(Vt, rnd(f["V"].T))
        off += (c2 * k * esz + 255) // 256 * 256 // esz
        Wrt = vals[off:off + c2 * c1].reshape(c2, c1)
        np.testing.assert_array_equal(Wrt, rnd(f["Wres"].T))


def test_plan_pack_tiled_upt():
    """bf16 plans with k + r = 320 and c1 a multiple of 64 (the 160 x 320
    first-stage tile) hold [U | P]^T k-tile-major: c1 / 32 blocks of
    (k + r) x 32; fp32 plans of the same spec keep the row layout."""
    c1, c2, k, r = 384, 384, 256, 64
    spec = D.make_spec(synth.KIND_LOWRANK, c1, c2, r, k=k)
    f = D.prepare(_w(2, c1, c2), spec)
    UPt = np.concatenate([f["U"].T, f["P"].T])
    vals = synth.bf16_to_f64(D.plan_pack(spec, f, synth.DT_BF16).view(np.uint16))
    tiled = vals[:(k + r) * c1].reshape(c1 // 32, k + r, 32)
    for t in range(c1 // 32):
        np.testing.assert_array_equal(tiled[t], _bf16(UPt[:, 32 * t:32 * t + 32]))
    vals32 = D.plan_pack(spec, f, synth.DT_F32).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(vals32[:(k + r) * c1].reshape(k + r, c1), synth.round_f32(UPt))


def test_plan_pack_monarch_fragment_order():
    """Monarch bf16 plans hold B1 and P in MFMA fragment order: the 16-byte
    run of lane l + 32 g in step s of block a holds rows 16 s + 8 g .. + 7 of
    column l (P: of column 32 q + l, zero past r; r padded to 32 rows)."""
    m, r = 32, 40
    c = m * m
    spec = D.make_spec(synth.KIND_MONARCH, c, c, r, mblk=m)
    rng = np.random.default_rng(5)
    f = {"B1": rng.standard_normal((m, m, m)), "B2": rng.standard_normal((m, m, m)),
         "P": rng.standard_normal((c, r)), "Wres": rng.standard_normal((c, c))}
    vals = synth.bf16_to_f64(D.plan_pack(spec, f, synth.DT_BF16).view(np.uint16))
    b1 = vals[:m * m * m].reshape(m, 2, 2, m, 8)          # [a][s][g][l][e]
    want = _bf16(f["B1"]).reshape(m, 2, 2, 8, m).transpose(0, 1, 2, 4, 3)
    np.testing.assert_array_equal(b1, want)
    off = (m * m * m * 2 + 255) // 256 * 256 // 2
    nq = (r + 31) // 32
    pt = vals[off:off + nq * 32 * c].reshape(nq, m, 2, 2, 32, 8)   # [q][a][s][g][l][e]
    Ppad = np.zeros((c, nq * 32))
    Ppad[:, :r] = f["P"]
    want = _bf16(Ppad).reshape(m, 2, 2, 8, nq, 32).transpose(4, 0, 1, 2, 5, 3)
    np.testing.assert_array_equal(pt, want)


def test_bf16_rounding_of_pack_matches_generator_rounding():
    """Library rounding (fp64 -> fp32 -> bf16, RNE) equals the generator's."""
    rng = np.random.default_rng(3)
    c1, c2, k, r = 64, 64, 8, 8
    spec = D.make_spec(synth.KIND_LOWRANK, c1, c2, r, k=k)
    vals = rng.standard_normal((c1, c2)) * np.exp(rng.uniform(-20, 20, (c1, c2)))
    f = {"U": np.zeros((c1, k)), "V": np.zeros((k, c2)), "P": np.zeros((c1, r)), "Wres": vals}
    buf = D.plan_pack(spec, f, synth.DT_BF16).view(np.uint16)
    off = ((k + r) * c1 * 2 + 255) // 256 * 256 // 2
    off += (c2 * k * 2 + 255) // 256 * 256 // 2
    got = buf[off:off + c1 * c2].reshape(c2, c1)
    np.testing.assert_array_equal(got, synth.bf16_bits(vals.T))


# ---------------------------------------------------------------------------
# input-aware static start (dyra_prepare_input_aware) against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("c1,c2,k,r", [(64, 96, 16, 8), (96, 64, 24, 16)])
def test_prepare_input_aware_matches_oracle(mode, c1, c2, k, r):
    W = _w(c1 * 7 + c2, c1, c2)
    w = synth.scaled(synth.WORKLOADS["vitb_fc1"], c1=c1, c2=c2, k=k, r=r)
    Xc = synth.make_calibration(w, 300)
    spec = D.make_spec(synth.KIND_LOWRANK, c1, c2, r, k=k)
    f = D.prepare_input_aware(W, spec, Xc, mode, nthreads=4)
    o = O.prepare(W, O.KIND_LOWRANK, r, k=k, calib=(Xc, mode))
    np.testing.assert_allclose(f["U"] @ f["V"], o["W_hat"], atol=1e-9)
    # sqrt(sigma) split of the transformed weight: S U_f and V_f^T have equal column norms
    S = O.input_transform(Xc, mode)
    np.testing.assert_allclose(np.linalg.norm(S @ f["U"], axis=0), np.linalg.norm(f["V"], axis=1), rtol=1e-8)
    _check_common(f, o, W, r)


def test_prepare_input_aware_rejects_bad_arguments():
    import ctypes
    spec = D.make_spec(synth.KIND_LOWRANK, 64, 96, 8, k=16)
    W = _w(3, 64, 96)
    Xc = np.ones((10, 64))
    with pytest.raises(D.DyraError, match="EINVAL"):
        D.prepare_input_aware(W, spec, Xc, 3)                                   # unknown mode
    with pytest.raises(D.DyraError, match="EINVAL"):
        D.prepare_input_aware(W, spec, np.zeros((10, 64)), 1)                   # all-zero rows
    bad = Xc.copy()
    bad[2, 5] = np.nan
    with pytest.raises(D.DyraError, match="EINVAL"):
        D.prepare_input_aware(W, spec, bad, 2)                                  # non-finite rows
    mon = D.make_spec(synth.KIND_MONARCH, 64, 64, 8, mblk=8)
    with pytest.raises(D.DyraError, match="EINVAL"):
        D.prepare_input_aware(_w(4, 64, 64), mon, Xc, 1)                        # not low-rank
    hf = D.HostFactors()
    assert D.lib().dyra_prepare_input_aware(ctypes.byref(spec), D._dptr(W), D._dptr(Xc), 10, 1,
                                            ctypes.byref(hf), 1) == -1          # null outputs
    assert D.lib().dyra_prepare_input_aware(ctypes.byref(spec), D._dptr(W), D._dptr(Xc), 0, 1,
                                            ctypes.byref(hf), 1) == -2          # no rows


def test_prepare_blast_diagonal_couplings_match_oracle():
    c1, c2, nb, rb, r = 64, 512, 4, 8, 8
    W = _w(77, c1, c2)
    spec = D.make_spec(synth.KIND_BLAST_DIAG, c1, c2, r, nb=nb, rb=rb)
    f = D.prepare(W, spec, nthreads=4)
    assert f["S"].shape == (nb, nb, rb)
    o = O.prepare(W, O.KIND_BLAST_DIAG, r, nb=nb, rb=rb)
    g = {"U": f["Ub"], "V": f["Vb"], "S": np.stack([[np.diag(f["S"][i, j]) for j in range(nb)] for i in range(nb)])}
    np.testing.assert_allclose(O.blast_dense(g), o["W_hat"], atol=1e-9)
    _check_common(f, o, W, r)
    # the device plan stores the diagonals only: St[j][i][p] = S[i][j][p]
    assert D.plan_size(spec, synth.DT_BF16) < D.plan_size(D.make_spec(synth.KIND_BLAST, c1, c2, r, nb=nb, rb=rb),
                                                          synth.DT_BF16)
