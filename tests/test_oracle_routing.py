"""Pins for the oracle's routing: brute force, a second route to the gates,
invariants of the permutation, and a hand-worked golden example."""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as orc
import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(L, k):
    T, E = L.shape
    idx = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))
        idx[t] = order[:k]
    return idx


@pytest.mark.parametrize("T,E,k,seed", [(64, 8, 2, 1), (200, 16, 4, 7), (50, 5, 5, 3), (33, 1, 1, 0)])
def test_topk_brute_force(T, E, k, seed):
    L = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    r = orc.route(L, k)
    assert np.array_equal(r.idx, _brute_topk(L, k))


def test_topk_ties_smaller_id_wins():
    # bf16-valued logits with many exact ties
    rng = np.random.default_rng(5)
    L = (rng.integers(-3, 4, size=(300, 16)) * 0.5).astype(np.float32)
    r = orc.route(L, 4)
    assert np.array_equal(r.idx, _brute_topk(L, 4))
    # all-equal row: experts 0..k-1, equal gates
    L2 = np.zeros((3, 8), dtype=np.float32)
    r2 = orc.route(L2, 3)
    assert np.array_equal(r2.idx, np.tile(np.arange(3), (3, 1)))
    assert np.allclose(r2.gate, 1.0 / 3.0, rtol=0, atol=1e-16)


@pytest.mark.parametrize("seed", [0, 1])
def test_gates_full_softmax_then_renormalise(seed):
    T, E, k = 100, 16, 4
    L = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32) * 3
    r = orc.route(L, k)
    Ld = L.astype(np.float64)
    p = np.exp(Ld - Ld.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, r.idx.astype(np.int64), axis=1)
    g2 = sel / sel.sum(axis=1, keepdims=True)
    assert np.max(np.abs(g2 - r.gate)) <= 1e-15
    assert np.allclose(r.gate.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # slot j holds the j-th largest gate
    assert np.all(np.diff(r.gate, axis=1) <= 0)


@pytest.mark.parametrize("cfg", [1, 3])
def test_permutation_invariants(cfg):
    d = mi.CONFIGS[cfg]
    if cfg == 3:  # keep the CPU suite small: same bias recipe at a reduced T
        d = mi.LayerDims(T=2048, H=64, I=32, E=128, k=8, dtype="bf16", skew=True)
    L = mi.make_inputs(d, seed=cfg, want=("logits",))["logits"]
    r = orc.route(L, d.k)
    M = d.T * d.k
    assert r.counts.sum() == M
    assert r.offsets[0] == 0 and r.offsets[-1] == M
    assert np.array_equal(np.sort(r.sorted_to_flat), np.arange(M))
    assert np.array_equal(r.flat_to_sorted[r.sorted_to_flat], np.arange(M))
    assert np.array_equal(r.sorted_to_flat[r.flat_to_sorted], np.arange(M))
    flat = r.idx.reshape(-1)
    for e in range(d.E):
        seg = r.sorted_to_flat[r.offsets[e]:r.offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)       # ascending token order inside a segment
    # a token's k experts are distinct
    assert all(len(set(row)) == d.k for row in r.idx.tolist())


def test_skewed_routing_shape():
    """The Zipf-biased logits give hot experts (> 5x mean) and empty experts."""
    d = mi.CONFIGS[3]
    L = mi.make_inputs(d, seed=3, want=("logits",))["logits"]
    r = orc.route(L, d.k)
    mean = d.T * d.k / d.E
    assert r.counts.max() > 5 * mean
    assert (r.counts == 0).sum() >= 1


def test_permute_then_unpermute_is_identity():
    d = mi.LayerDims(T=97, H=24, I=8, E=6, k=3, dtype="fp32")
    inp = mi.make_inputs(d, seed=11, want=("x", "logits"))
    r = orc.route(inp["logits"], d.k)
    x = inp["x"].astype(np.float64)
    Xp = x[r.sorted_to_flat // d.k]                    # permute
    back = Xp[r.flat_to_sorted].reshape(d.T, d.k, -1)  # unpermute
    assert np.array_equal(back.sum(axis=1), d.k * x * 1.0) or np.allclose(back.sum(axis=1), d.k * x)
    for j in range(d.k):
        assert np.array_equal(back[:, j], x)
    wsum = np.einsum("tk,tkh->th", r.gate, back)
    assert np.allclose(wsum, x, rtol=0, atol=1e-14)


def test_golden_routing_example():
    with open(os.path.join(GOLDEN, "routing_tiny.json")) as f:
        g = json.load(f)
    L = np.array(g["logits"], dtype=np.float32)
    r = orc.route(L, g["k"])
    assert r.idx.tolist() == g["idx"]
    assert np.allclose(r.gate, np.array(g["gate"]), rtol=0, atol=1e-15)
    assert r.counts.tolist() == g["counts"]
    assert r.offsets.tolist() == g["offsets"]
    assert r.sorted_to_flat.tolist() == g["sorted_to_flat"]
