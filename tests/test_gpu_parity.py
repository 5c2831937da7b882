"""GPU parity of the HIP layer against the fp64 oracle, through the C ABI.

Small shapes are compared element by element over every output; they span
several 128x128 GEMM tiles, ragged expert segments and an N tail.  Routing is
bit-exact; floating-point outputs must satisfy max|gpu-ref|/max|ref| <= 2e-2
for bf16 (the layer's stated tolerance) and <= 1e-4 for fp32.
"""
import numpy as np
import pytest

import grouped_gemm_layer_amd as gl
import moe_inputs as mi
from oracle import moe_oracle as orc
from _layer_harness import GpuRun, relerr, to_np, check_routing_exact, record_errors

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def _full_compare(dims, inp, tol):
    print(f"[parity] dims={dims}", flush=True)
    run = GpuRun(dims, inp)
    run.run_all()
    r = orc.route(inp["logits"], dims.k)
    check_routing_exact(run.routing_np(), r)
    Y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    g = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    L = run.layer
    errs = {
        "y": relerr(to_np(L.y), Y),
        "dx": relerr(to_np(L.dx), g["dx"]),
        "dw13": relerr(to_np(L.dw13), g["dw13"]),
        "dw2": relerr(to_np(L.dw2), g["dw2"]),
        "dgate": relerr(to_np(L.dgate), g["dgate"]),
        "dlogits": relerr(to_np(L.dlogits), g["dlogits"]),
    }
    record_errors(f"parity/{dims.run_mode}/T{dims.T}_H{dims.H}_I{dims.I}_E{dims.E}_k{dims.k}"
                  + ("_skew" if dims.skew else ""), errs, {k: tol for k in errs})
    for key, v in errs.items():
        assert v <= tol, (key, v)
    # empty experts have exactly zero weight gradients
    for e in np.nonzero(r.counts == 0)[0]:
        assert np.all(to_np(L.dw13[e]) == 0) and np.all(to_np(L.dw2[e]) == 0)
    return run, errs


def test_config1_fp32():
    d = mi.CONFIGS[1]
    _full_compare(d, mi.make_inputs(d, 1), TOL["fp32"])


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=300, H=256, I=128, E=8, k=2, dtype="bf16"), 101),
    (mi.LayerDims(T=1000, H=384, I=192, E=16, k=4, dtype="bf16"), 102),    # N tail (I=192)
    (mi.LayerDims(T=777, H=512, I=256, E=32, k=8, dtype="bf16", skew=True), 103),
    # the smallest H and I: the forward GEMMs (ping-pong loop) run a single
    # 64-wide K tile, the 256-column tiles are mostly tail
    (mi.LayerDims(T=500, H=64, I=64, E=8, k=2, dtype="bf16"), 104),
    # the 235B expert shape (both dgrad K dimensions >= 3072): the dgrad GEMMs
    # take their 256-row ping-pong tiles; experts of about 75 rows leave the
    # second wave row of every tile idle
    (mi.LayerDims(T=300, H=4096, I=1536, E=8, k=2, dtype="bf16"), 105),
])
def test_small_bf16(dims, seed):
    _full_compare(dims, mi.make_inputs(dims, seed), TOL["bf16"])


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=257, H=128, I=64, E=4, k=2, dtype="fp32"), 104),
    (mi.LayerDims(T=100, H=192, I=128, E=6, k=3, dtype="fp32", skew=True), 105),
])
def test_small_fp32(dims, seed):
    _full_compare(dims, mi.make_inputs(dims, seed), TOL["fp32"])


def test_edge_one_expert_k1():
    d = mi.LayerDims(T=129, H=128, I=64, E=1, k=1, dtype="bf16")
    _full_compare(d, mi.make_inputs(d, 106), TOL["bf16"])


def test_edge_all_tokens_to_one_expert():
    d = mi.LayerDims(T=400, H=128, I=128, E=8, k=1, dtype="bf16")
    inp = mi.make_inputs(d, 107)
    inp["logits"][:, 3] += 40.0
    run, _ = _full_compare(d, inp, TOL["bf16"])
    assert run.routing_np()["counts"].tolist() == [0, 0, 0, 400, 0, 0, 0, 0]


def test_wgrad_split_heavy_expert():
    """Experts with more rows than one weight-gradient chunk
    (moe_wgrad_chunk_rows, 8192): their dW13 and dW2 are summed from several
    chunks in chunk order.  Expert 0 takes every token (17000 rows: three
    chunks), expert 1 at least half of them (two chunks), the rest a few
    hundred each."""
    kc = gl.wgrad_chunk_rows()
    d = mi.LayerDims(T=17000, H=128, I=64, E=4, k=2, dtype="bf16")
    inp = mi.make_inputs(d, 111)
    inp["logits"][:, 0] += 4.0            # moderate biases: no gate underflows
    inp["logits"][: d.T // 2, 1] += 2.0
    run, _ = _full_compare(d, inp, TOL["bf16"])
    c = run.routing_np()["counts"]
    assert c[0] > 2 * kc and c[1] > kc


@pytest.mark.parametrize("dims,seed", [
    (mi.LayerDims(T=300, H=128, I=64, E=8, k=2, dtype="fp32"), 112),
    (mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True), 113),
    (mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True, mode="fp8_bwd"), 114),
    (mi.LayerDims(T=17000, H=128, I=64, E=4, k=2, dtype="bf16"), 115),   # split experts
])
def test_backward_accumulate_into(dims, seed):
    """moe_backward_accumulate adds the weight gradients to what dw13 / dw2
    hold: against the plain backward's result G and a random start R, an
    expert in one chunk gives R + G exactly (one fp32 add per element; empty
    experts keep R), a split expert (R + chunk 0) + chunk 1 ... within fp32
    rounding; every other output is bitwise that of the plain backward.  And
    against the oracle: (result - R) matches the oracle's dW13 and dW2 within
    the mode's bar (bf16 2e-2; fp8_bwd: the quantised oracle's bar, and
    against the exact backward 6e-2 or the definition's own error plus that
    bar, whichever is larger)."""
    import torch
    inp = mi.make_inputs(dims, seed)
    if dims.T == 17000:
        inp["logits"][:, 0] += 4.0
        inp["logits"][: dims.T // 2, 1] += 2.0
    print(f"[accumulate] dims={dims}", flush=True)
    run = GpuRun(dims, inp)
    run.run_all()
    L = run.layer
    G13, G2 = L.dw13.clone(), L.dw2.clone()
    others = [t.clone() for t in (L.dx, L.dgate, L.dlogits)]
    gen = torch.Generator(device="cuda").manual_seed(seed)
    R13 = torch.randn(G13.shape, device="cuda", generator=gen) * G13.abs().max()
    R2 = torch.randn(G2.shape, device="cuda", generator=gen) * G2.abs().max()
    L.dw13.copy_(R13)
    L.dw2.copy_(R2)
    run.layer.backward(run.dy, run.x, run.w13, run.w2, accumulate=True)
    torch.cuda.synchronize()
    for a, b in zip((L.dx, L.dgate, L.dlogits), others):
        assert torch.equal(a, b)
    counts = run.routing_np()["counts"]
    kc = gl.wgrad_chunk_rows()
    for got, R, G in ((L.dw13, R13, G13), (L.dw2, R2, G2)):
        for e in range(dims.E):
            if counts[e] <= kc:
                assert torch.equal(got[e], R[e] + G[e]), e
            else:
                err = (got[e] - (R[e] + G[e])).abs().max().item()
                assert err <= 1e-5 * (R[e].abs().max().item() + G[e].abs().max().item()), (e, err)
    # the accumulated gradients against the oracle
    r = orc.route(inp["logits"], dims.k)
    Y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    exact = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    added = {"dw13": to_np(L.dw13) - to_np(R13), "dw2": to_np(L.dw2) - to_np(R2)}
    tag = f"accumulate/{dims.run_mode}/T{dims.T}_E{dims.E}_k{dims.k}"
    if dims.run_mode == "fp8_bwd":
        from test_gpu_mxfp8 import TOL_EXACT, TOL_QORACLE
        quant = orc.backward_mxfp8(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
        e_q = {k: relerr(v, quant[k]) for k, v in added.items()}
        e_x = {k: relerr(v, exact[k]) for k, v in added.items()}
        bars_x = {k: max(TOL_EXACT, relerr(quant[k], exact[k]) + TOL_QORACLE[k]) for k in added}
        record_errors(tag + "/vs_quantised", e_q, TOL_QORACLE)
        record_errors(tag + "/vs_exact", e_x, bars_x)
        for k in added:
            assert e_q[k] <= TOL_QORACLE[k] and e_x[k] <= bars_x[k], (k, e_q[k], e_x[k])
    else:
        tol = TOL["fp32"] if dims.run_mode == "fp32" else TOL["bf16"]
        errs = {k: relerr(v, exact[k]) for k, v in added.items()}
        record_errors(tag, errs, {k: tol for k in errs})
        for k, v in errs.items():
            assert v <= tol, (k, v)


def test_edge_single_token():
    d = mi.LayerDims(T=1, H=64, I=64, E=4, k=2, dtype="bf16")
    _full_compare(d, mi.make_inputs(d, 108), TOL["bf16"])


def test_edge_logit_ties_route_exact():
    """bf16-valued logits with many ties at the top-k boundary: indices are bit-exact."""
    d = mi.LayerDims(T=2048, H=64, I=64, E=64, k=8, dtype="bf16")
    inp = mi.make_inputs(d, 109)
    inp["logits"] = np.round(inp["logits"] * 2.0).astype(np.float32) / 2.0
    run = GpuRun(d, inp)
    run.route()
    r = orc.route(inp["logits"], d.k)
    check_routing_exact(run.routing_np(), r)


def test_determinism_bitwise():
    d = mi.LayerDims(T=600, H=256, I=128, E=8, k=4, dtype="bf16", skew=True)
    inp = mi.make_inputs(d, 110)
    run = GpuRun(d, inp)
    outs = []
    for _ in range(2):
        run.run_all()
        L = run.layer
        outs.append([t.clone() for t in (L.y, L.dx, L.dw13, L.dw2, L.dgate, L.dlogits)] +
                    [getattr(L.routing, n).clone() for n in ("topk_idx", "gate", "sorted_to_flat")])
    import torch
    for a, b in zip(*outs):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("T,E,k,ties,seed", [
    (3000, 512, 32, False, 120),   # 8 logits per lane, 24 scan blocks (a full and a partial batch of 16)
    (3000, 512, 32, True, 121),    # the same with many ties at the top-k boundary
    (5000, 96, 5, False, 122),     # lanes 32..63 hold one logit
    (700, 8, 8, True, 123),        # k = E < 64: most lanes hold none
    (2000, 130, 8, True, 124),     # k <= 8 path: quarters of 33 experts, the last one 31, scalar loads
])
def test_route_extremes_exact(T, E, k, ties, seed):
    """Routing at the ends of the supported range (E up to 512, k up to 32)
    matches the oracle bit for bit: the wave arg-max over (value, expert)
    pairs (k > 8), the four-lanes-per-token selection (k <= 8) and the batched
    expert scan."""
    d = mi.LayerDims(T=T, H=64, I=64, E=E, k=k, dtype="bf16")
    print(f"[parity] route T={T} E={E} k={k} ties={ties}", flush=True)
    inp = mi.make_inputs(d, seed)
    if ties:
        inp["logits"] = np.round(inp["logits"] * 2.0).astype(np.float32) / 2.0
    run = GpuRun(d, inp)
    run.route()
    check_routing_exact(run.routing_np(), orc.route(inp["logits"], d.k))


def test_leftover_error_not_blamed_on_the_library():
    """An error left by an earlier, unrelated HIP call (an invalid device id)
    is neither reported by a valid library call nor cleared by it: the
    library reports the status of its own launches."""
    import ctypes
    import torch
    d = mi.LayerDims(T=256, H=128, I=64, E=8, k=2, dtype="bf16")
    inp = mi.make_inputs(d, 130)
    run = GpuRun(d, inp)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipGetLastError()                               # start from a clean state
    assert hip.hipSetDevice(100000) != 0                # leaves an error behind
    run.route()                                          # raises unless the call returns MOE_OK
    torch.cuda.synchronize()
    assert hip.hipGetLastError() != 0                    # still there for its owner
    assert hip.hipGetLastError() == 0
    check_routing_exact(run.routing_np(), orc.route(inp["logits"], d.k))
