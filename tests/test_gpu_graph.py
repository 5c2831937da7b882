"""The C ABI enqueues only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so route + forward + backward can be
captured in a HIP graph.  The graph is replayed several times, with eager
work and synchronisations in between and every output poisoned before each
replay; each replay must reproduce the eager results bit for bit (the layer
is deterministic)."""
import numpy as np
import pytest

import moe_inputs as mi
from _layer_harness import GpuRun

pytestmark = pytest.mark.gpu


def _outputs(L):
    return [L.y, L.dx, L.dw13, L.dw2, L.dgate, L.dlogits, L.routing.topk_idx, L.routing.gate,
            L.routing.sorted_to_flat, L.routing.flat_to_sorted, L.routing.offsets]


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True), 401),
    (mi.LayerDims(T=300, H=256, I=128, E=8, k=2, dtype="bf16", mode="fp8_bwd"), 402),
    (mi.LayerDims(T=500, H=256, I=128, E=8, k=4, dtype="bf16", skew=True, mode="mxfp8"), 403),
])
def test_graph_replays_match_eager(dims, seed):
    import torch
    print(f"[graph] dims={dims}", flush=True)
    run = GpuRun(dims, mi.make_inputs(dims, seed))
    run.run_all()
    L = run.layer
    eager = [t.clone() for t in _outputs(L)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up on the capture stream's side
        run.route(); run.forward(); run.backward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.route(); run.forward(); run.backward()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in _outputs(L):               # poison every output eagerly
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        scratch = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(L), eager)):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), (rep, i)
        del scratch


def test_graph_router_projection_replays_match_eager():
    """route_project + forward + backward + router_backward captured in one
    graph: every replay reproduces the eager logits, routing, layer outputs
    and router gradient bit for bit."""
    import torch
    dims = mi.LayerDims(T=500, H=256, I=128, E=16, k=4, dtype="bf16")
    print(f"[graph] router projection dims={dims}", flush=True)
    run = GpuRun(dims, mi.make_inputs(dims, 404))
    L = run.layer
    rng = np.random.default_rng(405)
    wr = torch.from_numpy(mi.bf16_round(rng.standard_normal((dims.E, dims.H)).astype(np.float32) * 0.05)).to(
        "cuda", torch.bfloat16)
    dwr = torch.empty((dims.E, dims.H), dtype=torch.float32, device="cuda")

    def step():
        L.route_project(run.x, wr)
        run.forward()
        run.backward()
        L.router_backward(run.x, wr, dwr)

    step()
    torch.cuda.synchronize()
    outs = lambda: _outputs(L) + [L.logits, dwr]
    eager = [t.clone() for t in outs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs():
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs(), eager)):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), (rep, i)


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True), 406),
    (mi.LayerDims(T=500, H=256, I=128, E=8, k=4, dtype="bf16", mode="mxfp8"), 407),
])
def test_graph_checkpointed_step_replays_match_eager(dims, seed):
    """The activation-checkpointing sequence (route, forward keeping no state,
    recompute, backward) captured in one graph: every replay reproduces the
    eager outputs of a plain route + forward + backward bit for bit, with the
    saved state poisoned before each replay."""
    import torch
    print(f"[graph] checkpointed step dims={dims}", flush=True)
    run = GpuRun(dims, mi.make_inputs(dims, seed))
    run.run_all()
    L = run.layer
    eager = [t.clone() for t in _outputs(L)]

    def step():
        run.route()
        L.forward(run.x, run.w13, run.w2, keep_saved=False)
        L.forward_recompute(run.x, run.w13, run.w2)
        run.backward()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in _outputs(L):
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        L.saved.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(L), eager)):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), (rep, i)
