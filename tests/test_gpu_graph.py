"""The forward captured in a HIP graph: replays, with eager work and host
synchronisation between them, give the eager forward's output bit for bit.
(The library launches only kernels on the caller's stream, so a caller may
capture it; the benchmark times such replays.)"""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth

from gpu_cases import host_factors_from_oracle, log, oracle_prepare

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
sc = synth.scaled


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    D.lib()


CASES = [
    sc(W["vitl_fc1"], name="graph_lowrank", B=6, s=300, c1=512, c2=1024, k=128, r=64),
    sc(W["monarch"], name="graph_monarch", B=3, s=200),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_graph_replay_matches_eager(w):
    import torch
    inp = synth.make_inputs(w)
    prep = oracle_prepare(w, inp.W)
    layer = D.DyraLayer(D.spec_of(w), host_factors_from_oracle(prep), w.dtype, bias=inp.bias)
    X = D.to_device(inp.X, w.dtype)
    Y = torch.empty((w.n, w.c2), dtype=D.torch_dtype(w.dtype), device="cuda")
    layer.workspace(w.B, w.s)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(X, w.B, w.s, out=Y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(X, w.B, w.s, out=Y)
    torch.cuda.synchronize()
    for rep in range(4):
        ref = layer.forward(X, w.B, w.s)        # eager work between the replays
        torch.cuda.synchronize()
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(Y, ref))
        log(f"  {w.name} replay {rep}: bitwise equal to eager = {same}")
        assert same
