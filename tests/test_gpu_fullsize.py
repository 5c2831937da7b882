"""GPU parity at the full layer shapes (Qwen3-30B-A3B and Qwen3-235B-A22B
expert shapes, T=16384, E=128, top-8), in the launch configuration the
benchmark times, compared with the fp64 oracle over every element.

Routing is compared bit-exactly.  y, dX, dW13, dW2, dgate and dlogits are
compared whole: max|gpu - ref| / max|ref| per tensor against the bf16 bar
2e-2, and the weight gradients of every empty expert must be exactly zero.
The Euler identities <dW2,W2> = <dW3,W3> = <dgate,gate> = <dY,Y> and the
zero row-sum of dlogits are checked as properties that hold at any size.
"""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as orc
from _layer_harness import GpuRun, relerr, to_np, check_routing_exact, record_errors, exact_layer

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_fullsize_whole(cfg):
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

    # properties over every output, in float64 on the device
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
    empty = np.nonzero(r.counts == 0)[0]
    for e in empty:
        assert torch.count_nonzero(L.dw13[int(e)]).item() == 0 and torch.count_nonzero(L.dw2[int(e)]).item() == 0

    # the whole layer through the oracle
    ref, _ = exact_layer(d, cfg, inp, r)
    errs = {"y": relerr(to_np(L.y), ref["y"])}
    for key, t in (("dx", L.dx), ("dgate", L.dgate), ("dlogits", L.dlogits), ("dw2", L.dw2), ("dw13", L.dw13)):
        errs[key] = relerr(to_np(t), ref[key])
    record_errors(f"fullsize/config{cfg}", errs, {k: TOL for k in errs})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
