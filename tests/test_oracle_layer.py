"""Pins for the oracle's layer forward and backward.

Each check compares the oracle with something other than itself:
  * torch (CPU, float64) autograd through a dense, permutation-free form of
    the layer (every token through every expert, weighted by the masked,
    renormalised softmax);
  * the dense SwiGLU FFN that the layer reduces to with one expert of weight 1;
  * central finite differences of the oracle's own forward;
  * the Euler identities (Y is homogeneous of degree 1 in W2, in W3 and in
    the gates) and the zero-sum of the softmax Jacobian;
  * a hand-worked golden example.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as orc
import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle_all(inp, k):
    r = orc.route(inp["logits"], k)
    Y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    g = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    return r, Y, g


def _torch_dense(inp, k):
    """Permutation-free layer in torch float64: Y = sum_e gbar[t,e] FFN_e(x[t])."""
    x = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
    w13 = torch.tensor(inp["w13"], dtype=torch.float64, requires_grad=True)
    w2 = torch.tensor(inp["w2"], dtype=torch.float64, requires_grad=True)
    L = torch.tensor(inp["logits"], dtype=torch.float64, requires_grad=True)
    dy = torch.tensor(inp["dy"], dtype=torch.float64)
    E = w13.shape[0]
    I = w13.shape[1] // 2
    p = torch.softmax(L, dim=-1)
    top = torch.topk(L.detach(), k, dim=-1).indices
    mask = torch.zeros_like(p).scatter_(1, top, 1.0)
    pm = p * mask
    gbar = pm / pm.sum(dim=-1, keepdim=True)
    gleaf = gbar.detach().clone().requires_grad_(True)   # for dL/dgate
    Y = torch.zeros_like(x)
    Yg = torch.zeros_like(x)
    for e in range(E):
        h = F.silu(F.linear(x, w13[e, :I])) * F.linear(x, w13[e, I:])
        o = F.linear(h, w2[e])
        Y = Y + gbar[:, e:e + 1] * o
        Yg = Yg + gleaf[:, e:e + 1] * o.detach()
    (Y * dy).sum().backward()
    (Yg * dy).sum().backward()
    return {"y": Y.detach().numpy(), "dx": x.grad.numpy(), "dw13": w13.grad.numpy(),
            "dw2": w2.grad.numpy(), "dlogits": L.grad.numpy(), "dgate_full": gleaf.grad.numpy(),
            "top": top.numpy()}


def _relerr(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(np.asarray(b))), 1e-300)


@pytest.mark.parametrize("dims,seed", [
    (mi.CONFIGS[1], 1),
    (mi.LayerDims(T=40, H=32, I=16, E=5, k=3, dtype="fp32"), 4),
    (mi.LayerDims(T=30, H=32, I=32, E=4, k=4, dtype="bf16"), 9),     # k = E
])
def test_oracle_matches_torch_autograd(dims, seed):
    inp = mi.make_inputs(dims, seed)
    r, Y, g = _oracle_all(inp, dims.k)
    ref = _torch_dense(inp, dims.k)
    assert np.array_equal(np.sort(r.idx, axis=1), np.sort(ref["top"], axis=1))
    assert _relerr(Y, ref["y"]) < 1e-12
    for key in ("dx", "dw13", "dw2", "dlogits"):
        assert _relerr(g[key], ref[key]) < 1e-11, key
    dgate_ref = np.take_along_axis(ref["dgate_full"], r.idx.astype(np.int64), axis=1)
    assert _relerr(g["dgate"], dgate_ref) < 1e-12


def test_one_expert_is_dense_swiglu_ffn():
    d = mi.LayerDims(T=50, H=64, I=32, E=1, k=1, dtype="fp32")
    inp = mi.make_inputs(d, 21)
    r, Y, _ = _oracle_all(inp, 1)
    x = torch.tensor(inp["x"], dtype=torch.float64)
    W1 = torch.tensor(inp["w13"][0, :32], dtype=torch.float64)
    W3 = torch.tensor(inp["w13"][0, 32:], dtype=torch.float64)
    W2 = torch.tensor(inp["w2"][0], dtype=torch.float64)
    dense = ((F.silu(x @ W1.T) * (x @ W3.T)) @ W2.T).numpy()
    assert _relerr(Y, dense) < 1e-13


def test_dominant_expert_with_k1_is_dense_ffn():
    d = mi.LayerDims(T=50, H=64, I=32, E=8, k=1, dtype="fp32")
    inp = mi.make_inputs(d, 22)
    inp["logits"][:, 5] += 30.0
    r, Y, _ = _oracle_all(inp, 1)
    assert np.all(r.idx[:, 0] == 5) and np.all(r.gate == 1.0)
    x = torch.tensor(inp["x"], dtype=torch.float64)
    W1 = torch.tensor(inp["w13"][5, :32], dtype=torch.float64)
    W3 = torch.tensor(inp["w13"][5, 32:], dtype=torch.float64)
    W2 = torch.tensor(inp["w2"][5], dtype=torch.float64)
    dense = ((F.silu(x @ W1.T) * (x @ W3.T)) @ W2.T).numpy()
    assert _relerr(Y, dense) < 1e-13


def test_k_equals_E_brute_force():
    d = mi.LayerDims(T=20, H=32, I=16, E=4, k=4, dtype="fp32")
    inp = mi.make_inputs(d, 23)
    r, Y, _ = _oracle_all(inp, 4)
    x = torch.tensor(inp["x"], dtype=torch.float64)
    p = torch.softmax(torch.tensor(inp["logits"], dtype=torch.float64), -1)
    ref = torch.zeros_like(x)
    for e in range(4):
        W1 = torch.tensor(inp["w13"][e, :16], dtype=torch.float64)
        W3 = torch.tensor(inp["w13"][e, 16:], dtype=torch.float64)
        W2 = torch.tensor(inp["w2"][e], dtype=torch.float64)
        ref += p[:, e:e + 1] * ((F.silu(x @ W1.T) * (x @ W3.T)) @ W2.T)
    assert _relerr(Y, ref.numpy()) < 1e-13


def test_finite_differences_config1():
    d = mi.CONFIGS[1]
    inp = {kk: v.astype(np.float64) for kk, v in mi.make_inputs(d, 1).items()}
    r, Y, g = _oracle_all(inp, d.k)
    dy = inp["dy"]

    def loss(x=None, w13=None, w2=None, L=None, gate=None):
        x = inp["x"] if x is None else x
        w13 = inp["w13"] if w13 is None else w13
        w2 = inp["w2"] if w2 is None else w2
        if gate is not None:
            Yp, _ = orc.forward_with_gates(x, w13, w2, r.idx, gate)
        else:
            rr = orc.route(inp["logits"] if L is None else L, d.k)
            Yp, _ = orc.forward(x, w13, w2, rr)
        return float(np.sum(dy * Yp))

    h = 1e-6
    rng = np.random.default_rng(0)
    checks = []
    for name, arr, key in (("x", inp["x"], "dx"), ("w13", inp["w13"], "dw13"),
                           ("w2", inp["w2"], "dw2"), ("gate", r.gate, "dgate"),
                           ("L", inp["logits"], "dlogits")):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if name == "L":
                # stay away from a change of the top-k set
                row = np.sort(arr[pos[0]])[::-1]
                if row[d.k - 1] - row[d.k] < 10 * h:
                    continue
            p = arr.copy(); p[pos] += h
            m = arr.copy(); m[pos] -= h
            fd = (loss(**{name: p}) - loss(**{name: m})) / (2 * h)
            an = g[key][pos]
            checks.append((name, fd, an))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)
    assert len(checks) >= 25


def test_euler_identities_and_router_zero_sum():
    d = mi.LayerDims(T=256, H=64, I=32, E=16, k=4, dtype="bf16")
    inp = mi.make_inputs(d, 31)
    r, Y, g = _oracle_all(inp, d.k)
    I = d.I
    dyY = float(np.sum(inp["dy"].astype(np.float64) * Y))
    w2 = inp["w2"].astype(np.float64)
    w3 = inp["w13"][:, I:].astype(np.float64)
    assert abs(np.sum(g["dw2"] * w2) - dyY) < 1e-10 * abs(dyY)
    assert abs(np.sum(g["dw13"][:, I:] * w3) - dyY) < 1e-10 * abs(dyY)
    assert abs(np.sum(g["dgate"] * r.gate) - dyY) < 1e-10 * abs(dyY)
    assert np.max(np.abs(g["dlogits"].sum(axis=1))) < 1e-13
    off = np.ones_like(g["dlogits"], dtype=bool)
    np.put_along_axis(off, r.idx.astype(np.int64), False, axis=1)
    assert np.all(g["dlogits"][off] == 0.0)


def test_empty_expert_has_zero_weight_gradient():
    d = mi.LayerDims(T=64, H=32, I=16, E=6, k=2, dtype="fp32")
    inp = mi.make_inputs(d, 41)
    inp["logits"][:, 2] -= 50.0          # nobody picks expert 2
    r, Y, g = _oracle_all(inp, d.k)
    assert r.counts[2] == 0
    assert np.all(g["dw13"][2] == 0) and np.all(g["dw2"][2] == 0)


def test_golden_expert_example():
    with open(os.path.join(GOLDEN, "expert_tiny.json")) as f:
        gd = json.load(f)
    inp = {kk: np.array(gd[kk], dtype=np.float64) for kk in ("x", "w13", "w2", "logits", "dy")}
    r, Y, g = _oracle_all(inp, gd["k"])
    assert np.allclose(Y, gd["y"], rtol=1e-14, atol=0)
    for key in ("dx", "dw13", "dw2", "dgate"):
        assert np.allclose(g[key], gd[key], rtol=1e-14, atol=1e-15), key


def test_router_projection_finite_differences():
    """Router projection (R13): L(x, W_r) = <dY, layer(x, route(x W_r^T))>.
    Central differences in x (which reaches the loss through the experts and
    through the logits) and in W_r pin dx = dx_experts + dlogits W_r and
    dW_r = dlogits^T x."""
    d = mi.CONFIGS[1]
    inp = {kk: v.astype(np.float64) for kk, v in mi.make_inputs(d, 1).items()}
    rng = np.random.default_rng(5)
    wr = rng.standard_normal((d.E, d.H)) * 0.1
    dy = inp["dy"]

    def loss(x, w):
        rr = orc.route(orc.router_logits(x, w), d.k)
        Yp, _ = orc.forward(x, inp["w13"], inp["w2"], rr)
        return float(np.sum(dy * Yp))

    logits = orc.router_logits(inp["x"], wr)
    r = orc.route(logits, d.k)
    _, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    g = orc.backward(dy, inp["x"], inp["w13"], inp["w2"], r, st)
    pr = orc.router_projection_backward(g["dlogits"], inp["x"], wr)
    dx = g["dx"] + pr["dx"]
    # the projection's own pieces against the definition of a matrix product
    assert np.allclose(logits, np.einsum("th,eh->te", inp["x"], wr), rtol=0, atol=1e-12)
    h = 1e-6
    margin = np.sort(logits, axis=1)[:, ::-1]
    margin = margin[:, d.k - 1] - margin[:, d.k]
    checks = 0
    for name, arr, an_full in (("x", inp["x"], dx), ("w", wr, pr["dw_router"])):
        for _ in range(8):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            toks = [pos[0]] if name == "x" else range(d.T)
            # a perturbation must not change any token's top-k set
            if min(margin[t] for t in toks) < 1e3 * h * (np.abs(wr).max() + np.abs(inp["x"]).max()):
                continue
            p = arr.copy(); p[pos] += h
            m = arr.copy(); m[pos] -= h
            fd = (loss(p, wr) - loss(m, wr)) / (2 * h) if name == "x" else \
                (loss(inp["x"], p) - loss(inp["x"], m)) / (2 * h)
            an = an_full[pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)
            checks += 1
    assert checks >= 10
    # the router's share of dx is not negligible here (the pin would miss a dropped term)
    assert np.abs(pr["dx"]).max() > 1e-3 * np.abs(g["dx"]).max()


def test_threaded_experts_give_the_same_arrays():
    """workers > 1 only schedules the independent experts on threads: every
    output of forward, backward and the quantised backward is bitwise the
    single-threaded one."""
    d = mi.LayerDims(T=300, H=128, I=64, E=8, k=2, dtype="bf16", skew=True)
    inp = mi.make_inputs(d, 21)
    r = orc.route(inp["logits"], d.k)
    Y1, s1 = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    Y4, s4 = orc.forward(inp["x"], inp["w13"], inp["w2"], r, workers=4)
    assert np.array_equal(Y1, Y4) and all(np.array_equal(s1[k], s4[k]) for k in s1)
    b1 = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, s1)
    b4 = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, s1, workers=4)
    q1 = orc.backward_mxfp8(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, s1)
    q4 = orc.backward_mxfp8(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, s1, workers=4)
    for a, b in ((b1, b4), (q1, q4)):
        assert all(np.array_equal(a[k], b[k]) for k in a)
    m1, _ = orc.forward_mxfp8(inp["x"], inp["w13"], inp["w2"], r)
    m4, _ = orc.forward_mxfp8(inp["x"], inp["w13"], inp["w2"], r, workers=4)
    assert np.array_equal(m1, m4)
