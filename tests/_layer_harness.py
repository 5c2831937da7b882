"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
layer through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import moe_inputs as mi


def relerr(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def to_dev(a: np.ndarray, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda", dtype=dtype)


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


class GpuRun:
    """Runs route / forward / backward of one shape on the GPU."""

    def __init__(self, dims: mi.LayerDims, inp: dict):
        import torch
        import grouped_gemm_layer_amd as g
        self.g = g
        self.dims = dims
        mode = dims.run_mode
        self.layer = g.MoeLayer(dims.T, dims.H, dims.I, dims.E, dims.k, mode=mode)
        adt = self.layer.act_dtype
        self.x = to_dev(inp["x"], adt)
        self.w13 = to_dev(inp["w13"], adt)
        self.w2 = to_dev(inp["w2"], adt)
        self.logits = to_dev(inp["logits"], torch.float32)
        self.dy = to_dev(inp["dy"], adt) if "dy" in inp else None

    def route(self):
        self.layer.route(self.logits)

    def forward(self):
        return self.layer.forward(self.x, self.w13, self.w2)

    def backward(self, want_dlogits=True):
        return self.layer.backward(self.dy, self.x, self.w13, self.w2, want_dlogits=want_dlogits)

    def run_all(self):
        import torch
        self.route()
        self.forward()
        self.backward()
        torch.cuda.synchronize()

    def routing_np(self) -> dict:
        r = self.layer.routing
        return {k: getattr(r, k).cpu().numpy() for k in
                ("topk_idx", "gate", "counts", "offsets", "sorted_to_flat", "flat_to_sorted")}


def check_routing_exact(gpu_r: dict, ref) -> None:
    assert np.array_equal(gpu_r["topk_idx"], ref.idx), "topk indices differ"
    assert np.array_equal(gpu_r["counts"], ref.counts), "counts differ"
    assert np.array_equal(gpu_r["offsets"], ref.offsets), "offsets differ"
    assert np.array_equal(gpu_r["sorted_to_flat"], ref.sorted_to_flat), "sorted_to_flat differs"
    assert np.array_equal(gpu_r["flat_to_sorted"], ref.flat_to_sorted), "flat_to_sorted differs"
    g = gpu_r["gate"].astype(np.float64)
    assert np.max(np.abs(g - ref.gate) / np.abs(ref.gate)) <= 1e-6, "gates differ"


# ---------------------------------------------------------------------------
# Sampled oracle evaluations for full-size shapes (rows are independent in the
# forward and in the activation-gradient chain; weight gradients need all rows
# of one expert).
# ---------------------------------------------------------------------------
def oracle_token_rows(orc, inp: dict, r, tokens) -> dict:
    """Y, dX, dgate, dlogits of the given tokens, from the oracle's per-expert functions."""
    k = r.k
    x, w13, w2, dy = inp["x"], inp["w13"], inp["w2"], inp["dy"]
    H = x.shape[1]
    Y = np.zeros((len(tokens), H))
    dX = np.zeros((len(tokens), H))
    dgate = np.zeros((len(tokens), k))
    for a, t in enumerate(tokens):
        for j in range(k):
            e = int(r.idx[t, j])
            g = r.gate[t, j]
            f = orc.expert_forward(x[t:t + 1], w13[e], w2[e])
            Y[a] += g * f["O"][0]
            dgate[a, j] = float(np.dot(dy[t].astype(np.float64), f["O"][0]))
            b = orc.expert_backward(g * dy[t:t + 1].astype(np.float64), x[t:t + 1], w13[e], w2[e], f)
            dX[a] += b["dX"][0]
    dlog = orc.router_backward(r.gate[tokens], dgate, r.idx[tokens], r.E)
    return {"y": Y, "dx": dX, "dgate": dgate, "dlogits": dlog}


def oracle_expert_wgrad(orc, inp: dict, r, e: int) -> dict:
    a, b = int(r.offsets[e]), int(r.offsets[e + 1])
    w13, w2 = inp["w13"], inp["w2"]
    if b == a:
        return {"dw13": np.zeros(w13.shape[1:]), "dw2": np.zeros(w2.shape[1:])}
    flat = r.sorted_to_flat[a:b]
    tok = flat // r.k
    g = r.gate.reshape(-1)[flat]
    f = orc.expert_forward(inp["x"][tok], w13[e], w2[e])
    bw = orc.expert_backward(g[:, None] * inp["dy"][tok].astype(np.float64), inp["x"][tok], w13[e], w2[e], f)
    return {"dw13": bw["dW13"], "dw2": bw["dW2"]}


def oracle_token_rows_mx8(orc, inp: dict, r, tokens, fwd=None) -> dict:
    """y, dX, dgate, dlogits of the given tokens under the fp8_bwd backward
    (fwd = the oracle's per-expert forward: expert_forward for fp8_bwd,
    expert_forward_mxfp8 for the mxfp8 mode).

    Row-wise quantisation (along H and 2I) treats each row on its own, so the
    rows of the sampled tokens are evaluated expert by expert with the
    oracle's per-expert fp8_bwd function (its weight gradients, which depend
    on all rows of the expert, are not used here)."""
    fwd = fwd or orc.expert_forward
    k = r.k
    x, w13, w2, dy = inp["x"], inp["w13"], inp["w2"], inp["dy"]
    H = x.shape[1]
    Y = np.zeros((len(tokens), H))
    dX = np.zeros((len(tokens), H))
    dgate = np.zeros((len(tokens), k))
    by_e = {}
    for a, t in enumerate(tokens):
        for j in range(k):
            by_e.setdefault(int(r.idx[t, j]), []).append((a, int(t), j))
    for e, rows in by_e.items():
        toks = np.array([t for _, t, _ in rows])
        g = np.array([r.gate[t, j] for _, t, j in rows])
        f = fwd(x[toks], w13[e], w2[e])
        out = orc.expert_backward_mxfp8(dy[toks], x[toks], g, w13[e], w2[e], f)
        for i, (a, t, j) in enumerate(rows):
            Y[a] += g[i] * f["O"][i]
            dX[a] += out["dXp"][i]
            dgate[a, j] = out["dgate"][i]
    dlog = orc.router_backward(r.gate[tokens], dgate, r.idx[tokens], r.E)
    return {"y": Y, "dx": dX, "dgate": dgate, "dlogits": dlog}


def oracle_expert_wgrad_mx8(orc, inp: dict, r, e: int, fwd=None) -> dict:
    """Weight gradients of expert e under the fp8_bwd backward (all of its rows)."""
    fwd = fwd or orc.expert_forward
    a, b = int(r.offsets[e]), int(r.offsets[e + 1])
    w13, w2 = inp["w13"], inp["w2"]
    if b == a:
        return {"dw13": np.zeros(w13.shape[1:]), "dw2": np.zeros(w2.shape[1:])}
    flat = r.sorted_to_flat[a:b]
    tok = flat // r.k
    g = r.gate.reshape(-1)[flat]
    f = fwd(inp["x"][tok], w13[e], w2[e])
    out = orc.expert_backward_mxfp8(inp["dy"][tok], inp["x"][tok], g, w13[e], w2[e], f)
    return {"dw13": out["dW13"], "dw2": out["dW2"]}
