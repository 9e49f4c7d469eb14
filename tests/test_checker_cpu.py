"""The GPU parity checker (tests/gpu_cases.py) can see the mistakes a
whole-output Frobenius ratio cannot: at the ViT-L fc1 shape the correction
L R is about 5 % of ||Y||, so one segment without its correction, or one
zeroed 256 x 128 output tile, moves the whole-output ratio by less than the
2e-2 bar.  Everything here runs on the CPU from the oracle alone: an output
with the bf16 rounding of the first-stage product T and of Y applied (the
storage points the GPU rounds at) must pass, and the same output with one
planted mistake must fail."""
import numpy as np
import pytest

from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O

from gpu_cases import oracle_prepare, oracle_terms, parity_report, rounded_prep

W = synth.WORKLOADS
sc = synth.scaled

# ViT-L fc1 layer shape (c1, c2, k, r and the input law of the full
# workload), four of its 32 segments
VITL4 = sc(W["vitl_fc1"], name="vitl_fc1_4seg", B=4)


@pytest.fixture(scope="module")
def vitl4():
    w = VITL4
    inp = synth.make_inputs(w)
    rp = rounded_prep(oracle_prepare(w, inp.W), w.dtype)
    terms = oracle_terms(w, inp.X, rp, inp.bias)
    f = rp["static"]
    T = synth.round_bf16(inp.X @ f["U"])
    Y_like = synth.round_bf16(T @ f["V"] + terms[1] + inp.bias)   # bf16 T and Y, exact correction
    return w, inp, rp, terms, Y_like


@pytest.mark.parametrize("kind", [O.KIND_LOWRANK, O.KIND_MONARCH, O.KIND_BLAST])
@pytest.mark.parametrize("t", [1.0, 1.5, 2.0])
def test_terms_sum_to_the_oracle_forward(kind, t):
    base = {O.KIND_LOWRANK: sc(W["vitb_fc1"], B=3, s=40, c1=64, c2=96, k=16, r=8),
            O.KIND_MONARCH: sc(W["monarch"], B=2, s=50, c1=1024, c2=1024, r=16),
            O.KIND_BLAST: sc(W["lm_blast"], B=2, s=60, c1=128, c2=256, nb=4, rb=8, r=8, n_out=2)}[kind]
    inp = synth.make_inputs(base)
    rp = rounded_prep(oracle_prepare(base, inp.W), base.dtype)
    Y, corr, mag, _ = oracle_terms(base, inp.X, rp, inp.bias, eps=1e-6, t=t)
    assert np.array_equal(Y, O.forward(inp.X, rp, inp.bias, base.B, base.s, eps=1e-6, t=t))
    assert np.all(mag >= np.abs(Y) * (1 - 1e-12))


def test_checker_accepts_storage_rounding(vitl4):
    w, _, _, terms, Y_like = vitl4
    m, fails = parity_report(w, Y_like, terms)
    assert not fails, fails
    # the premise: the correction is a small share of Y at this shape
    assert 0.02 < m["corr_share"] < 0.1


def test_whole_output_ratio_misses_what_the_checker_finds(vitl4):
    w, _, _, terms, Y_like = vitl4
    Y, corr, _, _ = terms
    s = w.s
    dropped = Y_like.copy()
    dropped[2 * s:3 * s] -= corr[2 * s:3 * s]                  # segment 2 without L R
    tile = Y_like.copy()
    tile[s + 300:s + 556, 1024:1152] = 0.0                     # one 256 x 128 output tile
    for bad in (dropped, tile):
        m, fails = parity_report(w, bad, terms)
        # spread over the workload's 32 segments the same mistake moves the
        # whole-output ratio by sqrt(4 / 32) of what it moves here: under 2e-2
        assert m["rel_fro"] * np.sqrt(w.B / 32) < 2e-2
        assert any(f.startswith("segment") for f in fails), fails


def test_checker_separates_t_1p5_from_t_1(vitl4):
    """An output with one ALS iteration fails against the t = 1.5 oracle."""
    w, inp, rp, terms, Y_like = vitl4
    terms15 = oracle_terms(w, inp.X, rp, inp.bias, t=1.5)
    m, fails = parity_report(w, Y_like, terms15)
    assert fails
    # and the t = 1.5 output in the same storage rounding passes
    T = synth.round_bf16(inp.X @ rp["static"]["U"])
    Y15 = synth.round_bf16(T @ rp["static"]["V"] + terms15[1] + inp.bias)
    m, fails = parity_report(w, Y15, terms15)
    assert not fails, fails


def test_checker_still_sees_a_dropped_correction_on_an_ill_conditioned_segment():
    """A segment with as many tokens as r has cond(L_b) in the hundreds, so it
    gets the conditioning allowance; without its correction it still fails."""
    w = sc(W["vitb_fc1"], name="ill", B=1, s=982, c1=256, c2=264, k=32, r=16)
    off = [0, 437, 453, 982]                                # segment 1: 16 = r tokens
    inp = synth.make_inputs(w)
    rp = rounded_prep(oracle_prepare(w, inp.W), w.dtype)
    terms = oracle_terms(w, inp.X, rp, inp.bias, offsets=off)
    Y, corr, _, conds = terms
    assert 2.0 ** -8 * conds[1] > 0.25 and 2.0 ** -8 * conds[0] < 0.25
    ok = synth.round_bf16(Y)
    m, fails = parity_report(w, ok, terms, offsets=off)
    assert not fails and m["ill_conditioned_segments"] == 1, fails
    bad = ok.copy()
    bad[437:453] -= corr[437:453]
    m, fails = parity_report(w, bad, terms, offsets=off)
    assert any(f.startswith("segment 1") for f in fails), fails
