"""The seeded shapes of the GPU shape sweep satisfy the library's host-side
validation (plan and workspace sizes are accepted), so the sweep never sends
the device a shape the library would reject; no GPU needed."""
import importlib.util
import os

import numpy as np

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _sweep_module():
    spec = importlib.util.spec_from_file_location("shape_sweep", os.path.join(HERE, "test_gpu_shape_sweep.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_sweep_shapes_pass_host_validation():
    m = _sweep_module()
    for w in m.SHAPES + m.STRUCTURED:
        sp = D.spec_of(w)
        assert D.plan_size(sp, w.dtype) > 0, w.name
        assert D.workspace_size(sp, w.B, w.s, w.dtype) > 0, w.name
        assert w.s >= w.r, w.name
    for w, off in m.RAGGED:
        sp = D.spec_of(w)
        assert off[0] == 0 and off[-1] == w.s and np.all(np.diff(off) >= 1), w.name
        assert D.workspace_size_varlen(sp, off, w.dtype) > 0, w.name


def test_sweep_is_deterministic():
    a, b = _sweep_module(), _sweep_module()
    assert [(w.B, w.s, w.c1, w.c2, w.k, w.r, w.dtype, w.bias) for w in a.SHAPES] == \
           [(w.B, w.s, w.c1, w.c2, w.k, w.r, w.dtype, w.bias) for w in b.SHAPES]
