"""GPU parity at the full layer shapes (Qwen3-30B-A3B and Qwen3-235B-A22B
expert shapes, T=16384, E=128, top-8), in the launch configuration the
benchmark times.

Routing is compared bit-exactly in full.  The fp64 oracle cannot run the
whole layer here in seconds, so it evaluates sampled outputs one by one:
Y, dX, dgate and dlogits of sampled tokens (rows are independent), and the
weight gradients of sampled experts (the most loaded one, a median one and,
with skewed routing, an empty one).  Properties that hold at any size are
checked over every output: the Euler identities <dW2,W2> = <dW3,W3> =
<dgate,gate> = <dY,Y> and the zero row-sum of dlogits.
"""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as orc
from _layer_harness import (GpuRun, relerr, to_np, check_routing_exact, oracle_token_rows,
                            oracle_expert_wgrad)

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_fullsize_sampled(cfg):
    import torch
    d = mi.CONFIGS[cfg]
    print(f"[fullsize] config {cfg}: {mi.CONFIG_NAMES[cfg]}", flush=True)
    inp = mi.make_inputs(d, cfg)
    run = GpuRun(d, inp)
    run.run_all()
    L = run.layer
    r = orc.route(inp["logits"], d.k)
    check_routing_exact(run.routing_np(), r)
    if cfg == 3:
        mean = d.M / d.E
        assert r.counts.max() > 5 * mean and (r.counts == 0).sum() >= 1
        print(f"[fullsize] skew: max/mean {r.counts.max() / mean:.1f}, empty experts "
              f"{int((r.counts == 0).sum())}", flush=True)

    rng = np.random.default_rng(1000 + cfg)
    tokens = np.unique(np.concatenate([rng.choice(d.T, 30, replace=False), [0, d.T - 1]]))
    ref = oracle_token_rows(orc, inp, r, tokens)
    tt = torch.as_tensor(tokens, device="cuda")
    errs = {
        "y": relerr(to_np(L.y[tt]), ref["y"]),
        "dx": relerr(to_np(L.dx[tt]), ref["dx"]),
        "dgate": relerr(to_np(L.dgate[tt]), ref["dgate"]),
        "dlogits": relerr(to_np(L.dlogits[tt]), ref["dlogits"]),
    }
    order = np.argsort(r.counts, kind="stable")
    experts = [int(order[-1]), int(order[d.E // 2])]
    if (r.counts == 0).any():
        experts.append(int(np.nonzero(r.counts == 0)[0][0]))
    for e in experts:
        w = oracle_expert_wgrad(orc, inp, r, e)
        if r.counts[e] == 0:
            assert torch.count_nonzero(L.dw13[e]).item() == 0 and torch.count_nonzero(L.dw2[e]).item() == 0
            continue
        errs[f"dw13[{e}]"] = relerr(to_np(L.dw13[e]), w["dw13"])
        errs[f"dw2[{e}]"] = relerr(to_np(L.dw2[e]), w["dw2"])
    print("[fullsize] sampled errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)

    # Euler identities over all outputs, in float64 on the device
    f64 = torch.float64
    I = d.I
    dyY = torch.sum(run.dy.to(f64) * L.y.to(f64)).item()
    w2w = torch.sum(L.dw2.to(f64) * run.w2.to(f64)).item()
    w3w = torch.sum(L.dw13[:, I:].to(f64) * run.w13[:, I:].to(f64)).item()
    gg = torch.sum(L.dgate.to(f64) * L.routing.gate.to(f64)).item()
    print(f"[fullsize] Euler: dyY {dyY:.6e} dW2.W2 {w2w:.6e} dW3.W3 {w3w:.6e} dgate.g {gg:.6e}", flush=True)
    for v in (w2w, w3w, gg):
        assert abs(v - dyY) <= 2e-2 * abs(dyY)
    rowsum = L.dlogits.to(f64).sum(dim=1).abs().max().item()
    assert rowsum <= 1e-5 * L.dlogits.abs().max().item() * d.k
