"""GPU tests of the activation-checkpointing recompute (moe_forward_recompute):
after the saved state is overwritten, the recompute restores what the
backward reads, bit for bit, and leaves y alone."""
import numpy as np
import pytest

import moe_inputs as mi
from _layer_harness import GpuRun

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True), 601),
    (mi.LayerDims(T=300, H=128, I=64, E=8, k=2, dtype="fp32"), 602),
    (mi.LayerDims(T=700, H=384, I=192, E=16, k=4, dtype="bf16", mode="fp8_bwd"), 603),
    (mi.LayerDims(T=700, H=384, I=256, E=16, k=4, dtype="bf16", mode="mxfp8"), 604),
])
def test_recompute_restores_saved_bitwise(dims, seed):
    import torch
    print(f"[recompute] dims={dims}", flush=True)
    run = GpuRun(dims, mi.make_inputs(dims, seed))
    run.run_all()
    L = run.layer
    ref = [t.clone() for t in (L.dx, L.dw13, L.dw2, L.dgate, L.dlogits)]
    M = dims.T * dims.k
    g13_bytes = M * 2 * dims.I * (2 if dims.run_mode == "bf16" else 4)   # G13 is kept in fp32 in the fp8 modes
    saved_u8 = L.saved.view(torch.uint8)
    g13_ref = saved_u8[:g13_bytes].clone()
    saved_u8.fill_(0xFF)                      # NaN patterns in every element the backward could read
    y_u8 = L.y.view(torch.uint8)
    y_u8.fill_(0x5A)
    L.forward_recompute(run.x, run.w13, run.w2)
    torch.cuda.synchronize()
    assert torch.equal(saved_u8[:g13_bytes], g13_ref), "G13 differs after the recompute"
    assert bool((y_u8 == 0x5A).all()), "the recompute wrote y"
    run.backward()
    torch.cuda.synchronize()
    for name, a, b in zip(("dx", "dw13", "dw2", "dgate", "dlogits"), ref, (L.dx, L.dw13, L.dw2, L.dgate, L.dlogits)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True), 611),
    (mi.LayerDims(T=300, H=128, I=64, E=8, k=2, dtype="fp32"), 612),
    (mi.LayerDims(T=700, H=384, I=256, E=16, k=4, dtype="bf16", mode="mxfp8"), 614),
])
def test_forward_without_saved_state(dims, seed):
    """moe_forward with saved = NULL (checkpointing's first forward) gives the
    same y bit for bit and leaves the saved buffer untouched; a recompute then
    feeds the backward as a full forward would."""
    import torch
    print(f"[recompute] no-save dims={dims}", flush=True)
    run = GpuRun(dims, mi.make_inputs(dims, seed))
    run.run_all()
    L = run.layer
    y_ref = L.y.clone()
    ref = [t.clone() for t in (L.dx, L.dw13, L.dw2, L.dgate, L.dlogits)]
    saved_u8 = L.saved.view(torch.uint8)
    saved_u8.fill_(0x3C)
    L.y.zero_()
    L.forward(run.x, run.w13, run.w2, keep_saved=False)
    torch.cuda.synchronize()
    assert torch.equal(L.y.view(torch.uint8), y_ref.view(torch.uint8)), "y differs"
    assert bool((saved_u8 == 0x3C).all()), "the forward wrote the saved state"
    L.forward_recompute(run.x, run.w13, run.w2)
    run.backward()
    torch.cuda.synchronize()
    for name, a, b in zip(("dx", "dw13", "dw2", "dgate", "dlogits"), ref, (L.dx, L.dw13, L.dw2, L.dgate, L.dlogits)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name
