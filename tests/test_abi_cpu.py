"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments with the documented codes before touching the GPU (CPU only)."""
import ctypes

import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth


def test_library_exports_every_header_symbol():
    L = D.lib()
    names = D.header_symbols()
    assert len(names) >= 9
    for name in names:
        assert hasattr(L, name), name


def test_status_strings():
    L = D.lib()
    for code in D.ERRORS:
        assert L.dyra_status_string(code)
    assert L.dyra_status_string(0) == b"ok"


def _lowrank(c1=64, c2=96, k=16, r=8):
    return D.make_spec(synth.KIND_LOWRANK, c1, c2, r, k=k)


@pytest.mark.parametrize("spec,code", [
    (D.make_spec(synth.KIND_LOWRANK, 64, 96, 8, k=0), -2),        # k = 0
    (D.make_spec(synth.KIND_LOWRANK, 64, 96, 8, k=60), -2),       # k + r > min
    (D.make_spec(synth.KIND_LOWRANK, 64, 96, 12, k=16), -2),      # r not multiple of 8
    (D.make_spec(synth.KIND_LOWRANK, 60, 96, 8, k=16), -2),       # c1 not multiple of 8
    (D.make_spec(synth.KIND_LOWRANK, 512, 512, 136, k=16), -2),   # r > 128
    (D.make_spec(synth.KIND_MONARCH, 64, 64, 8, mblk=8), 0),
    (D.make_spec(synth.KIND_MONARCH, 64, 72, 8, mblk=8), -2),     # not square
    (D.make_spec(synth.KIND_BLAST, 64, 96, 8, nb=4, rb=8), 0),
    (D.make_spec(synth.KIND_BLAST, 64, 96, 8, nb=5, rb=8), -2),   # nb does not divide
    (D.make_spec(synth.KIND_BLAST, 64, 96, 8, nb=4, rb=32), -2),  # rb > block
    (D.make_spec(7, 64, 96, 8, k=16), -1),                        # unknown kind
])
def test_prepare_sizes_validation(spec, code):
    s = D.Sizes()
    assert D.lib().dyra_prepare_sizes(ctypes.byref(spec), ctypes.byref(s)) == code


def test_sizes_and_plan_and_workspace_sizes():
    spec = _lowrank()
    sz = D.prepare_sizes(spec)
    assert sz["U"] == 64 * 16 and sz["V"] == 16 * 96 and sz["P"] == 64 * 8 and sz["R0"] == 8 * 96
    assert sz["Wres"] == 64 * 96 and sz["B1"] == 0
    pb = D.plan_size(spec, synth.DT_BF16)
    pf = D.plan_size(spec, synth.DT_F32)
    assert pb >= 2 * ((16 + 8) * 64 + 96 * 16 + 96 * 64) and pf >= 2 * pb - 512 * 3
    w1 = D.workspace_size(spec, 2, 50, synth.DT_BF16)
    w2 = D.workspace_size(spec, 4, 50, synth.DT_BF16)
    assert 0 < w1 < w2


def test_dtype_support_matrix():
    L = D.lib()
    n = ctypes.c_size_t()
    mon = D.make_spec(synth.KIND_MONARCH, 1024, 1024, 64, mblk=32)
    assert L.dyra_plan_size(ctypes.byref(mon), synth.DT_BF16, ctypes.byref(n)) == 0
    assert L.dyra_plan_size(ctypes.byref(mon), synth.DT_F32, ctypes.byref(n)) == -6
    assert L.dyra_plan_size(ctypes.byref(mon), 5, ctypes.byref(n)) == -1


def _fwd(spec, plan=1 << 12, X=1 << 12, bias=None, Y=1 << 13, B=2, s=50, dtype=synth.DT_BF16, eps=1e-6,
         solver=0, ws=1 << 14, ws_bytes=None):
    """Calls dyra_forward with fake (never dereferenced) aligned addresses;
    every case below must be rejected on the host before any HIP call."""
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return D.lib().dyra_forward(ctypes.byref(spec), plan, X, bias, Y, B, s, dtype, eps, solver, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(plan=None), -1),
    (dict(X=None), -1),
    (dict(Y=None), -1),
    (dict(ws=None), -1),
    (dict(eps=-1.0), -1),
    (dict(eps=float("nan")), -1),
    (dict(solver=9), -1),
    (dict(dtype=3), -1),
    (dict(B=0), -2),
    (dict(s=0), -2),
    (dict(B=1 << 20, s=1 << 12), -2),
    (dict(X=(1 << 12) + 2), -1),          # misaligned
    (dict(bias=(1 << 15) + 4), -1),       # misaligned bias
    (dict(ws_bytes=16), -3),
])
def test_forward_rejects_bad_arguments_before_any_hip_call(kw, code):
    assert _fwd(_lowrank(), **kw) == code


def test_forward_rejects_bad_spec():
    bad = D.make_spec(synth.KIND_LOWRANK, 64, 96, 8, k=92)
    assert _fwd(bad) == -2


def test_dense_ref_validation():
    L = D.lib()
    assert L.dyra_dense_ref(None, 16, None, 32, 4, 8, 8, synth.DT_BF16, None) == -1
    assert L.dyra_dense_ref(16, 32, None, 64, 4, 7, 8, synth.DT_BF16, None) == -2
    assert L.dyra_dense_ref(16, 32, None, 64, 0, 8, 8, synth.DT_BF16, None) == -2
    assert L.dyra_dense_ref(16, 32, None, 64, 4, 8, 8, 2, None) == -1
    assert L.dyra_dense_ref(18, 32, None, 64, 4, 8, 8, synth.DT_BF16, None) == -1


def test_solver_status_validation():
    L = D.lib()
    out = np.zeros(2, np.int32)
    p = out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.dyra_solver_status(None, 16, 2, 4, synth.DT_BF16, p, None) == -1
    spec = _lowrank()
    assert L.dyra_solver_status(ctypes.byref(spec), None, 2, 4, synth.DT_BF16, p, None) == -1
    assert L.dyra_solver_status(ctypes.byref(spec), 16, 0, 4, synth.DT_BF16, p, None) == -2


def test_prepare_rejects_missing_outputs():
    spec = _lowrank()
    W = np.zeros((64, 96))
    hf = D.HostFactors()
    rc = D.lib().dyra_prepare(ctypes.byref(spec), W.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                              ctypes.byref(hf), 1)
    assert rc == -1


def test_als_entry_points_validate_on_host():
    """dyra_workspace_size_als / dyra_forward_als reject what they do not
    support before any HIP call: half_steps outside 2..4, a structure other
    than low-rank, fp32."""
    L = D.lib()
    lowrank = D.make_spec(synth.KIND_LOWRANK, 256, 512, 16, k=32)
    monarch = D.make_spec(synth.KIND_MONARCH, 1024, 1024, 16, mblk=32)
    n = ctypes.c_size_t()
    for h, rc in ((2, 0), (3, 0), (4, 0), (1, -1), (5, -1)):
        assert L.dyra_workspace_size_als(ctypes.byref(lowrank), 2, 64, synth.DT_BF16, h, ctypes.byref(n)) == rc
    assert L.dyra_workspace_size_als(ctypes.byref(lowrank), 2, 64, synth.DT_F32, 3, ctypes.byref(n)) == -6
    assert L.dyra_workspace_size_als(ctypes.byref(monarch), 2, 64, synth.DT_BF16, 3, ctypes.byref(n)) == -1
    sizes = []
    for h in (2, 3, 4):
        L.dyra_workspace_size_als(ctypes.byref(lowrank), 2, 64, synth.DT_BF16, h, ctypes.byref(n))
        sizes.append(n.value)
    base = ctypes.c_size_t()
    L.dyra_workspace_size(ctypes.byref(lowrank), 2, 64, synth.DT_BF16, ctypes.byref(base))
    assert sizes[0] == base.value and sizes[1] == sizes[2] > sizes[0]
    # forward: argument errors come back before any device work
    assert L.dyra_forward_als(ctypes.byref(lowrank), 16, 16, None, 16, 2, 64, synth.DT_BF16, 1e-6, 0, 7, 16,
                              1 << 30, None) == -1
    assert L.dyra_forward_als(ctypes.byref(lowrank), 16, 16, None, 16, 2, 64, synth.DT_F32, 1e-6, 0, 3, 16,
                              1 << 30, None) == -6
    assert L.dyra_forward_als(ctypes.byref(lowrank), 16, 16, None, 16, 2, 64, synth.DT_BF16, 1e-6, 0, 3, 16,
                              sizes[0], None) == -3
