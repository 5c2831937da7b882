"""The allocation-free routing entry point (moe_route_noalloc) against the
workspace one (moe_route), through the C ABI: two calls in a row, the second
on a smaller shape, each bit for bit equal to moe_route and to the oracle's
routing (indices, counts, offsets and both maps exact; gates within fp32
rounding of the fp64 softmax)."""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as orc
from _layer_harness import check_routing_exact, to_dev

pytestmark = pytest.mark.gpu


def _route_both(T, E, k, seed, ties):
    import torch
    import grouped_gemm_layer_amd as g
    d = g.Dims.of(T, 64, 64, E, k, "bf16")
    print(f"[noalloc] T={T} E={E} k={k} ties={ties}", flush=True)
    inp = mi.make_inputs(mi.LayerDims(T=T, H=64, I=64, E=E, k=k, dtype="bf16"), seed, want=("logits",))
    logits = inp["logits"]
    if ties:
        logits = np.round(logits * 2.0).astype(np.float32) / 2.0
    lt = to_dev(logits, torch.float32)
    rws = g.workspace_size(d)[0]
    ref = g.alloc_routing(d)
    g.route(d, lt, ref, g.alloc_workspace(rws))
    got = g.alloc_routing(d)
    for name in ("topk_idx", "gate", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        getattr(got, name).fill_(-7)                     # poison: every entry must be written
    g.route_noalloc(d, lt, got)
    torch.cuda.synchronize()
    for name in ("topk_idx", "gate", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        a, b = getattr(got, name), getattr(ref, name)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    check_routing_exact({n: getattr(got, n).cpu().numpy() for n in
                         ("topk_idx", "gate", "counts", "offsets", "sorted_to_flat", "flat_to_sorted")},
                        orc.route(logits, k))


def test_route_noalloc_two_calls_second_smaller():
    _route_both(16384, 128, 8, 501, False)     # 32 blocks of expert partials
    _route_both(700, 64, 4, 502, True)         # smaller: stale partials of the first call must not leak in


def test_route_noalloc_rejects_shapes_beyond_the_scratch():
    import torch
    import grouped_gemm_layer_amd as g
    d = g.Dims.of(131072, 64, 64, 512, 32, "bf16")   # 1024 blocks x 512 experts x 2 x 4 B = 4 MiB
    assert g.workspace_size(d)[0] > 2 << 20
    r = g.alloc_routing(g.Dims.of(1, 64, 64, 512, 32, "bf16"))
    lt = torch.zeros(1, 512, dtype=torch.float32, device="cuda")
    with pytest.raises(g.MoeError) as ei:
        g.route_noalloc(d, lt, r)
    assert ei.value.status == 5
