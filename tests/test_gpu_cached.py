"""Cached MXFP8 weights (the two fp8 modes): moe_quantize_weights once, then
moe_forward_cached / moe_backward_cached, through the C ABI.  Every output
must equal, bit for bit, that of moe_forward / moe_backward quantising the
same weights in the call (the same codes enter the same GEMMs), and the
results are therefore those the quantised and exact oracles already check
in test_gpu_mxfp8."""
import pytest

import moe_inputs as mi
from _layer_harness import GpuRun

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=300, H=256, I=128, E=8, k=2, dtype="bf16", mode="fp8_bwd"), 601),
    (mi.LayerDims(T=777, H=512, I=256, E=32, k=8, dtype="bf16", skew=True, mode="fp8_bwd"), 602),
    (mi.LayerDims(T=500, H=256, I=128, E=8, k=4, dtype="bf16", skew=True, mode="mxfp8"), 603),
    (mi.LayerDims(T=9000, H=256, I=128, E=4, k=2, dtype="bf16", mode="mxfp8"), 604),   # split weight gradients
])
def test_cached_weights_bitwise(dims, seed):
    import torch
    print(f"[cached] dims={dims}", flush=True)
    inp = mi.make_inputs(dims, seed)
    ref = GpuRun(dims, inp)
    ref.run_all()
    L = ref.layer
    want = [t.clone() for t in (L.y, L.dx, L.dw13, L.dw2, L.dgate, L.dlogits)]
    run = GpuRun(dims, inp)
    C = run.layer
    run.route()
    C.quantize_weights(run.w13, run.w2)
    for t in (C.y, C.dx, C.dw13, C.dw2, C.dgate, C.dlogits):
        t.fill_(float("nan"))                      # every output must be written
    C.forward_cached(run.x, run.w13, run.w2)
    C.backward_cached(run.dy, run.x)
    torch.cuda.synchronize()
    got = [C.y, C.dx, C.dw13, C.dw2, C.dgate, C.dlogits]
    for name, a, b in zip(("y", "dx", "dw13", "dw2", "dgate", "dlogits"), got, want):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name
