"""GPU parity over a seeded sweep of irregular low-rank layer shapes: odd
segment counts and lengths, ragged token and output-column counts, every
residual rank step from 8 to 128, with and without bias, bf16 and fp32.
Each shape picks its own kernel paths (first-stage tile or engine GEMM,
Gram partials from the first stage or their own launch, token split, the
right factor split over K or on the persistent kernel with one or several
tiles per workgroup, ...); every one is held to the same per-segment,
correction and elementwise checks as the fixed cases.  Run on an MI355X:
pytest -m gpu."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth

from gpu_cases import run_same_factor_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _shapes(count=24, seed=20261204):
    """Seeded shapes within the library's constraints (c1, c2, k, r
    multiples of 8, r <= 128, k + r <= min(c1, c2)); segments at least r
    tokens long (shorter ones have dedicated cases)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        c1 = 8 * int(rng.integers(8, 201))
        c2 = 8 * int(rng.integers(8, 201))
        m = min(c1, c2)
        r = 8 * int(rng.integers(1, min(16, m // 8 - 1) + 1))
        k = 8 * int(rng.integers(1, (m - r) // 8 + 1))
        if i % 6 == 0 and m >= 320 and r in (32, 64):
            k = 320 - r                       # the 160 x 320 first-stage tile
        B = int(rng.integers(1, 13))
        s = int(rng.integers(r, max(r + 1, 7200 // B)))
        dtype = synth.DT_F32 if i % 5 == 4 else synth.DT_BF16
        out.append(synth.scaled(W["vitl_fc1"], name=f"sweep{i:02d}", seed=5000 + i, B=B, s=s, c1=c1, c2=c2,
                                k=k, r=r, dtype=dtype, bias=bool(rng.integers(0, 2))))
    return out


SHAPES = _shapes()


def _structured(seed=20261205):
    """Seeded Monarch (c = 1024, blocks of 32; bf16) and BLAST shapes (nb
    dividing c1 and c2, c2 / nb a multiple of 128, rb <= min(c1, c2) / nb)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(4):
        r = 8 * int(rng.integers(1, 17))
        B = int(rng.integers(1, 10))
        s = int(rng.integers(r, 3000 // B + r))
        out.append(synth.scaled(W["monarch"], name=f"sweep_monarch{i}", seed=6000 + i, B=B, s=s, r=r,
                                bias=bool(rng.integers(0, 2))))
    for i in range(6):
        nb = int(rng.choice([2, 4, 8]))
        c2 = nb * 128 * int(rng.integers(1, 4))
        c1 = nb * 8 * int(rng.integers(4, 17))
        rb = 8 * int(rng.integers(1, min(c1, c2) // nb // 8 + 1))
        r = 8 * int(rng.integers(1, min(16, min(c1, c2) // 8 - 1) + 1))
        B = int(rng.integers(1, 6))
        s = int(rng.integers(r, 2000 // B + r))
        base = W["lm_blast_diag"] if i % 2 else W["lm_blast"]
        out.append(synth.scaled(base, name=f"sweep_blast{i}", seed=7000 + i, B=B, s=s, c1=c1, c2=c2, nb=nb,
                                rb=rb, r=r, solver="auto", bias=bool(rng.integers(0, 2))))
    return out


STRUCTURED = _structured()


def _ragged(seed=20261206):
    """Seeded ragged batches (lengths 1 .. 900) on a few low-rank shapes."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(5):
        c1 = 8 * int(rng.integers(16, 129))
        c2 = 8 * int(rng.integers(16, 129))
        r = 8 * int(rng.integers(1, 9))
        k = 8 * int(rng.integers(1, (min(c1, c2) - r) // 8 + 1))
        lengths = rng.integers(1, 900, size=int(rng.integers(2, 12)))
        off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        w = synth.scaled(W["vitl_fc1"], name=f"sweep_ragged{i}", seed=8000 + i, B=1, s=int(off[-1]), c1=c1,
                         c2=c2, k=k, r=r, dtype=synth.DT_F32 if i == 4 else synth.DT_BF16)
        out.append((w, off))
    return out


RAGGED = _ragged()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    D.lib()


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: f"{w.name}_B{w.B}s{w.s}_{w.c1}x{w.c2}_k{w.k}r{w.r}_"
                                                   f"{'bf16' if w.dtype == synth.DT_BF16 else 'f32'}")
def test_shape_sweep(w):
    err, status, _, _ = run_same_factor_case(w)
    assert np.all(status == D.SOLVE_OK)


@pytest.mark.parametrize("w", STRUCTURED, ids=lambda w: f"{w.name}_B{w.B}s{w.s}_{w.c1}x{w.c2}_r{w.r}"
                                                       + (f"_nb{w.nb}rb{w.rb}" if w.nb else ""))
def test_structured_sweep(w):
    err, status, _, _ = run_same_factor_case(w, solver=w.solver)
    assert np.all(status == D.SOLVE_OK)


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: f"{c[0].name}_{len(c[1]) - 1}seg_{c[0].c1}x{c[0].c2}"
                                                      f"_k{c[0].k}r{c[0].r}")
def test_ragged_sweep(case):
    w, off = case
    err, status, _, _ = run_same_factor_case(w, offsets=off)
    assert np.all(status == D.SOLVE_OK)


@pytest.mark.parametrize("w", SHAPES[:6], ids=lambda w: w.name)
def test_als_sweep(w):
    """t = 2 on the first six sweep shapes."""
    err, status, _, _ = run_same_factor_case(w, half_steps=4)
    assert np.all(status == D.SOLVE_OK)
