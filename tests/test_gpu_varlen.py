"""GPU parity of the forward over ragged segments (dyra_forward_varlen: one
ALS solve per segment of its own length, as for prompts of mixed length in
one prefill batch) against the float64 oracle, through the C-ABI; and the
uniform case through the ragged entry point, bit for bit dyra_forward."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth

from gpu_cases import gpu_forward, gpu_forward_varlen, host_factors_from_oracle, log, oracle_prepare, \
    run_same_factor_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
sc = synth.scaled


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    D.lib()


def _offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _mix(seed, B, lo, hi):
    """Seeded segment lengths, uniform in [lo, hi]."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=B)


CASES = [
    # one-row and shorter-than-r segments beside long ones (chunk Gram path)
    ("lowrank_mixed", sc(W["vitb_fc1"], c1=256, c2=264, k=32, r=16), [1, 300, 7, 129, 16, 450, 2, 77]),
    ("lowrank_mixed_fp32", sc(W["vitb_fc1"], c1=192, c2=200, k=24, r=16, dtype=synth.DT_F32), [3, 150, 64, 1, 90]),
    # k + r = 320 with every segment >= 160 rows: Gram partials from the
    # first-stage tile epilogue, tiles straddling ragged boundaries
    ("lowrank_tile_gram", sc(W["vitl_fc1"], c1=384, c2=512, k=256, r=64), list(_mix(7, 9, 160, 700))),
    ("lowrank_tile_short", sc(W["vitl_fc1"], c1=384, c2=512, k=256, r=64), [5, 400, 33, 250]),
    ("monarch_mixed", sc(W["monarch"], r=32), [11, 300, 1, 200, 97]),
    # few segments, long ones: the M strips split their tokens (2 parts; the
    # 37-token segment's second part is partial)
    ("lowrank_token_split", sc(W["vitl_fc1"], c1=512, c2=512, k=64, r=64), [1500, 37, 1100]),
    ("blast_mixed", sc(W["lm_blast"], c1=512, c2=1536, nb=4, rb=32, r=32, n_out=4, solver="auto"),
     [40, 1, 300, 111]),
    ("blast_diag_mixed", sc(W["lm_blast_diag"], c1=512, c2=1536, nb=4, rb=32, r=32, n_out=4, solver="auto"),
     [200, 13, 90]),
]


@pytest.mark.parametrize("name,base,lengths", CASES, ids=[c[0] for c in CASES])
def test_ragged_segments(name, base, lengths):
    off = _offsets(lengths)
    w = sc(base, name=name, B=1, s=int(off[-1]))     # inputs for all rows; segments from the offsets
    err, status, _, _ = run_same_factor_case(w, solver=w.solver, offsets=off)
    assert len(status) == len(lengths)
    assert np.all(status == D.SOLVE_OK)       # the ridge keeps even 1-row segments solvable


def test_ragged_prefill_mix_at_vitl_width():
    """A prefill-like batch at the ViT-L fc1 layer shape: 24 prompts of 64 ..
    2048 tokens (about 25k rows), every kernel on its full-size path."""
    lengths = _mix(11, 24, 64, 2048)
    off = _offsets(lengths)
    w = sc(W["vitl_fc1"], name="vitl_prefill_mix", B=1, s=int(off[-1]))
    log(f"  lengths {lengths.tolist()}")
    err, status, _, _ = run_same_factor_case(w, offsets=off)
    assert np.all(status == D.SOLVE_OK)


@pytest.mark.parametrize("name,base,B,s", [
    ("uniform_lowrank", sc(W["vitl_fc1"], c1=384, c2=512, k=256, r=64), 5, 300),
    ("uniform_monarch", sc(W["monarch"], r=64), 3, 77),
])
def test_uniform_offsets_match_dyra_forward_bitwise(name, base, B, s):
    w = sc(base, name=name, B=B, s=s)
    inp = synth.make_inputs(w)
    f = host_factors_from_oracle(oracle_prepare(w, inp.W))
    (Y,), st = gpu_forward(w, f, inp.X, inp.bias)
    Yv, stv = gpu_forward_varlen(w, f, inp.X, inp.bias, np.arange(B + 1, dtype=np.int64) * s)
    assert np.array_equal(Y, Yv) and np.array_equal(st, stv)


# more ALS iterations on ragged segments: each segment's left step uses its
# own rows of X (the left-step GEMM reads the offsets)
ALS_CASES = [
    ("als_lowrank_mixed", sc(W["vitb_fc1"], c1=256, c2=264, k=32, r=16), [41, 300, 77, 129, 36, 450]),
    ("als_lowrank_fp32", sc(W["vitb_fc1"], c1=192, c2=200, k=24, r=16, dtype=synth.DT_F32), [150, 64, 31, 90]),
    ("als_tile_gram", sc(W["vitl_fc1"], c1=384, c2=512, k=256, r=64), [700, 160, 333, 900]),
    ("als_monarch", sc(W["monarch"], r=32), [300, 97, 200]),
    ("als_blast", sc(W["lm_blast"], c1=512, c2=1536, nb=4, rb=32, r=32, n_out=4, solver="auto"), [200, 113, 90]),
]


@pytest.mark.parametrize("half_steps", [3, 4])
@pytest.mark.parametrize("name,base,lengths", ALS_CASES, ids=[c[0] for c in ALS_CASES])
def test_ragged_segments_als(name, base, lengths, half_steps):
    off = _offsets(lengths)
    w = sc(base, name=name, B=1, s=int(off[-1]))
    err, status, _, _ = run_same_factor_case(w, solver=w.solver, offsets=off, half_steps=half_steps)
    assert np.all(status == D.SOLVE_OK)
