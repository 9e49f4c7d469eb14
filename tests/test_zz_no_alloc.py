"""The allocation-free forward (dyra_forward_noalloc, workspace in the
library's static device array) against dyra_forward with a caller-allocated
workspace, through the C-ABI: two calls in a row, the second on a smaller
input, each giving the same output bit for bit and the same solver status
words (the two entry points run the same kernels on the same inputs)."""
import numpy as np
import pytest

from input_adaptive_rank_amd import dyra as D
from input_adaptive_rank_amd import synth
from oracle import dyra_oracle as O

from gpu_cases import TOL, host_factors_from_oracle, log, oracle_prepare

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
sc = synth.scaled


def test_noalloc_matches_forward_on_two_calls_in_a_row():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    big = sc(W["vitl_fc1"], name="noalloc_first", B=4, s=257, c1=256, c2=512, k=64, r=64)
    small = sc(big, name="noalloc_second_smaller", B=3, s=100)
    inp = synth.make_inputs(big)
    prep = oracle_prepare(big, inp.W)
    layer = D.DyraLayer(D.spec_of(big), host_factors_from_oracle(prep), big.dtype, bias=inp.bias)
    Xall = D.to_device(inp.X, big.dtype)
    for w in (big, small):
        X = Xall[:w.n].contiguous()
        log(f"  no-alloc call {w.name}: B={w.B} s={w.s} c1={w.c1} c2={w.c2} k={w.k} r={w.r}")
        ref = layer.forward(X, w.B, w.s)
        torch.cuda.synchronize()
        ref_status = layer.status(w.B, w.s)
        Y = torch.full((w.n, w.c2), float("nan"), dtype=D.torch_dtype(w.dtype), device=X.device)
        st = torch.full((w.B,), -7, dtype=torch.int32, device=X.device)
        D.forward_noalloc(layer.spec, layer.plan, X, layer.bias, Y, w.B, w.s, w.dtype, status=st)
        torch.cuda.synchronize()
        a = Y.float().cpu().numpy().astype(np.float64)
        b = ref.float().cpu().numpy().astype(np.float64)
        err = O.rel_fro(a, b)
        log(f"    rel_fro vs dyra_forward {err:.3e}, bitwise equal {bool(torch.equal(Y, ref))}, "
            f"status {st.cpu().tolist()} / {ref_status.tolist()}")
        assert err <= TOL[w.dtype]
        assert torch.equal(Y, ref)
        assert np.array_equal(st.cpu().numpy(), ref_status)
