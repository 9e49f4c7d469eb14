"""Seeded synthetic inputs for the DyRA layer forward.

This module is shared by the tests, the benchmark and the oracle-side checks.
It holds only input construction (random draws, orthogonal factors, spectra,
storage rounding); none of the method's arithmetic lives here.

Workloads stand in for the activations and weights of the models the DyRA
paper evaluates (no dataset item or trained weight is used):
  * ViT-B/16 at 224 px: 197 tokens per image, MLP fc1 768 -> 3072.
  * ViT-L/16 (DINOv3-like, 512 px): 1024 patches + CLS + 4 registers = 1029
    tokens per image, MLP 1024 -> 4096 (fc1) and 4096 -> 1024 (fc2).
  * LM prefill: one 4096-token prompt, hidden 4096, fused QKV width 12288.

Recipe (all float64, numpy PCG64 via default_rng(seed)), draws in this order:
  1. outlier channel indices: rng.choice(c1, n_out, replace=False)
  2. Z (n x c1): standard normal, or Student-t(4)/sqrt(2) for heavy tails
  3. G1 (c1 x m) -> U = QR, columns sign-fixed by sign(diag R)  (Haar)
  4. G2 (c2 x m) -> V likewise
  5. bias: 0.02 * standard normal (when the workload has a bias)
  X = Z diag(sigma), sigma_i = i^-0.7 (1-based), outlier channels x20.
  W = U diag(s) V^T, s_i = i^-0.5, m = min(c1, c2).
Storage rounding: bf16 workloads hold values that are exactly representable
in bf16 (fp64 -> fp32 round-to-nearest-even -> bf16 round-to-nearest-even);
the fp32 workload holds fp32-representable values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

KIND_LOWRANK = 0
KIND_MONARCH = 1
KIND_BLAST = 2
KIND_BLAST_DIAG = 3

DT_F32 = 0
DT_BF16 = 1


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int              # segments (images / sequences)
    s: int              # rows (tokens) per segment
    c1: int             # input features
    c2: int             # output features
    kind: int           # KIND_*
    r: int              # residual (dynamic) rank
    k: int = 0          # low-rank static rank
    mblk: int = 0       # Monarch: number of blocks == block size
    nb: int = 0         # BLAST: nb x nb block grid
    rb: int = 0         # BLAST: shared-basis rank
    dtype: int = DT_BF16
    bias: bool = True
    n_out: int = 4      # outlier channels
    heavy_tail: bool = False
    solver: str = "auto"
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def n(self) -> int:
        return self.B * self.s


# The five layer shapes of the DyRA layer-forward workloads.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1001, 1, 256, 256, 256, KIND_LOWRANK, 8, k=64,
                          dtype=DT_F32, bias=False),
    "vitb_fc1": Workload("vitb_fc1", 1002, 64, 197, 768, 3072, KIND_LOWRANK, 32, k=192),
    "vitl_fc1": Workload("vitl_fc1", 1003, 32, 1029, 1024, 4096, KIND_LOWRANK, 64, k=256),
    "vitl_fc2": Workload("vitl_fc2", 1003, 32, 1029, 4096, 1024, KIND_LOWRANK, 64, k=256),
    "monarch": Workload("monarch", 1004, 32, 1029, 1024, 1024, KIND_MONARCH, 64, mblk=32),
    "lm_blast": Workload("lm_blast", 1005, 1, 4096, 4096, 12288, KIND_BLAST, 128, nb=16, rb=128,
                         n_out=16, heavy_tail=True, solver="ns"),
    # the same layer with diagonal couplings S_ij = diag(s_ij)
    "lm_blast_diag": Workload("lm_blast_diag", 1005, 1, 4096, 4096, 12288, KIND_BLAST_DIAG, 128, nb=16,
                              rb=128, n_out=16, heavy_tail=True, solver="ns"),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(changes)
    return Workload(**d)


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def bf16_bits(a) -> np.ndarray:
    """uint16 bf16 bit patterns of `a` (fp64 -> fp32 RNE -> bf16 RNE)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        rounded = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)
    return rounded


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """fp64 values that bf16 storage of `a` represents exactly."""
    return bf16_to_f64(bf16_bits(a))


def round_f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_storage(a, dtype: int) -> np.ndarray:
    return round_bf16(a) if dtype == DT_BF16 else round_f32(a)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def haar_columns(G: np.ndarray) -> np.ndarray:
    """Orthonormal columns from a Gaussian matrix (QR with sign(diag R) fix)."""
    Q, R = np.linalg.qr(G)
    d = np.sign(np.diag(R))
    d[d == 0] = 1.0
    return Q * d


def channel_scales(c1: int, outliers: np.ndarray, alpha: float = 0.7,
                   outlier_scale: float = 20.0) -> np.ndarray:
    sigma = np.arange(1, c1 + 1, dtype=np.float64) ** (-alpha)
    sigma[outliers] *= outlier_scale
    return sigma


@dataclass
class Inputs:
    X: np.ndarray           # n x c1, fp64 holding storage-representable values
    W: np.ndarray           # c1 x c2, fp64 (storage-rounded)
    bias: np.ndarray | None
    W_exact: np.ndarray     # c1 x c2 fp64 before storage rounding
    spectrum: np.ndarray    # singular values used to build W_exact


def make_inputs(w: Workload, n_rows: int | None = None) -> Inputs:
    """Draw X, W and bias for a workload, in the fixed order of the recipe.

    n_rows, when given, draws only the first n_rows rows of Z (same seed, so
    a prefix of the full X is reproduced exactly since Z is drawn row-major).
    """
    rng = np.random.default_rng(w.seed)
    c1, c2 = w.c1, w.c2
    outliers = rng.choice(c1, w.n_out, replace=False) if w.n_out > 0 else np.zeros(0, int)
    n = w.n if n_rows is None else n_rows
    if w.heavy_tail:
        Z = rng.standard_t(4.0, size=(w.n, c1)) / np.sqrt(2.0)
    else:
        Z = rng.standard_normal((w.n, c1))
    Z = Z[:n]
    m = min(c1, c2)
    U = haar_columns(rng.standard_normal((c1, m)))
    V = haar_columns(rng.standard_normal((c2, m)))
    s = np.arange(1, m + 1, dtype=np.float64) ** (-0.5)
    W_exact = (U * s) @ V.T
    bias = 0.02 * rng.standard_normal(c2) if w.bias else None
    X = Z * channel_scales(c1, outliers)
    return Inputs(X=round_storage(X, w.dtype), W=round_storage(W_exact, w.dtype),
                  bias=None if bias is None else round_storage(bias, w.dtype),
                  W_exact=W_exact, spectrum=s)


def make_calibration(w: Workload, n_cal: int) -> np.ndarray:
    """n_cal calibration rows from the workload's input law: the same outlier
    channels and channel scales as make_inputs (drawn from the same seed),
    rows from an independent stream (seed + 1000003), storage-rounded."""
    rng = np.random.default_rng(w.seed)
    outliers = rng.choice(w.c1, w.n_out, replace=False) if w.n_out > 0 else np.zeros(0, int)
    rz = np.random.default_rng(w.seed + 1000003)
    if w.heavy_tail:
        Z = rz.standard_t(4.0, size=(n_cal, w.c1)) / np.sqrt(2.0)
    else:
        Z = rz.standard_normal((n_cal, w.c1))
    return round_storage(Z * channel_scales(w.c1, outliers), w.dtype)


def orthonormal_rows_input(rng: np.random.Generator, n: int, c1: int, scale: float = 1.0):
    """X with X^T X = scale^2 I (n >= c1): scaled Haar-orthonormal columns."""
    return scale * haar_columns(rng.standard_normal((n, c1)))
