"""Router projection (logits = x W_r^T) and its backward on the GPU against
the fp64 oracle (R13).  The top-k of the GPU's fp32 logits must equal the
oracle's top-k of those same fp32 values bit for bit (floating point decides
an integer there, so both sides decide on the same values); the logits
themselves, dx (experts' share plus the router's) and dW_r are compared
within tolerance."""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as orc
from _layer_harness import GpuRun, check_routing_exact, relerr, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL_LOGITS = 1e-5     # fp32 accumulation of H bf16 products against fp64
TOL = 2e-2            # bf16 outputs / gradients


def _router_weights(dims, seed):
    rng = np.random.default_rng(seed)
    return mi.bf16_round(rng.standard_normal((dims.E, dims.H)).astype(np.float32) * 0.05)


def _run(dims, seed, bias=None):
    import torch
    print(f"[router] dims={dims} seed={seed}", flush=True)
    inp = mi.make_inputs(dims, seed)
    wr = _router_weights(dims, seed + 1000)
    if bias is not None:
        # steer the routing through the projection: a constant feature column
        # of x times a large router weight favours the chosen experts
        inp["x"][:, 0] = 1.0
        wr[:, 0] = mi.bf16_round(np.asarray(bias, dtype=np.float32))
    run = GpuRun(dims, inp)
    L = run.layer
    wr_d = to_dev(wr, torch.bfloat16)
    logits = L.route_project(run.x, wr_d)
    run.forward()
    run.backward()
    dx_layer = L.dx.clone()
    dwr = torch.full((dims.E, dims.H), float("nan"), dtype=torch.float32, device="cuda")
    L.router_backward(run.x, wr_d, dwr)
    torch.cuda.synchronize()
    return inp, wr, run, to_np(logits), to_np(dx_layer), to_np(L.dx), to_np(dwr)


@pytest.mark.parametrize("dims,seed,skew", [
    (mi.LayerDims(T=600, H=256, I=128, E=16, k=4, dtype="bf16"), 501, False),
    (mi.LayerDims(T=333, H=192, I=64, E=40, k=3, dtype="bf16"), 502, False),     # E and T off the tiles
    (mi.LayerDims(T=700, H=256, I=128, E=16, k=2, dtype="bf16"), 503, True),     # two experts take most rows
])
def test_router_projection_small(dims, seed, skew):
    bias = None
    if skew:
        bias = np.zeros(dims.E, dtype=np.float32)
        bias[[3, 11]] = 4.0
    inp, wr, run, logits, dx_layer, dx, dwr = _run(dims, seed, bias)
    x = inp["x"]
    ref_logits = orc.router_logits(x, wr)
    e_log = relerr(logits, ref_logits)
    r = orc.route(logits, dims.k)                      # the oracle's top-k of the GPU's fp32 logits
    check_routing_exact(run.routing_np(), r)
    Y, st = orc.forward(x, inp["w13"], inp["w2"], r)
    g = orc.backward(inp["dy"], x, inp["w13"], inp["w2"], r, st)
    pr = orc.router_projection_backward(g["dlogits"], x, wr)
    errs = {"logits": e_log, "y": relerr(to_np(run.layer.y), Y), "dx_layer": relerr(dx_layer, g["dx"]),
            "dx": relerr(dx, g["dx"] + pr["dx"]), "dw_router": relerr(dwr, pr["dw_router"])}
    print("[router] errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    if skew:
        c = run.routing_np()["counts"]
        assert c[3] + c[11] > dims.T, c
    assert errs["logits"] <= TOL_LOGITS
    for key in ("y", "dx_layer", "dx", "dw_router"):
        assert errs[key] <= TOL, (key, errs[key])
    # the router's share of dx is not negligible here
    assert np.abs(pr["dx"]).max() > 1e-2 * np.abs(g["dx"]).max()


def test_router_projection_fullsize_sampled():
    """The Qwen3-30B-A3B shape: logits of sampled tokens against fp64, the
    routing bit-exact on the GPU's logits, and the projection backward
    against fp64 evaluations from the GPU's own dlogits (the layer's dlogits
    are checked by the layer's parity tests): dx on sampled tokens, dW_r on
    sampled experts (the most loaded, a median one, the least loaded)."""
    dims = mi.CONFIGS[2]
    inp, wr, run, logits, dx_layer, dx, dwr = _run(dims, 504)
    x = inp["x"].astype(np.float64)
    rng = np.random.default_rng(7)
    toks = rng.choice(dims.T, size=48, replace=False)
    e_log = relerr(logits[toks], orc.router_logits(x[toks], wr))
    r = orc.route(logits, dims.k)
    check_routing_exact(run.routing_np(), r)
    dl = to_np(run.layer.dlogits)
    e_dx = relerr(dx[toks], dx_layer[toks] + dl[toks] @ wr.astype(np.float64))
    order = np.argsort(r.counts)
    experts = [int(order[-1]), int(order[dims.E // 2]), int(order[0])]
    e_dw = max(relerr(dwr[e], dl[:, e] @ x) for e in experts)
    print(f"[router] fullsize logits {e_log:.2e} dx {e_dx:.2e} dw_router {e_dw:.2e}", flush=True)
    assert e_log <= TOL_LOGITS
    assert e_dx <= TOL
    assert e_dw <= 1e-4          # fp32 sums of the same products, no bf16 rounding on the way
