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


def record_errors(test: str, errs: dict, bars: dict) -> None:
    """Print the achieved per-tensor errors of a parity test next to its bars
    (one line, kept in the pytest output) and, when MOE_PARITY_RECORD names a
    file, append them there as one JSON line."""
    import json
    import os
    rec = {"test": test, "errors": {k: float(v) for k, v in errs.items()},
           "bars": {k: float(bars[k]) for k in errs if k in bars}}
    print("[parity-record]", json.dumps(rec), flush=True)
    path = os.environ.get("MOE_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


# The exact fp64 layer (oracle forward and backward) of full-size inputs,
# computed once per test process: the bf16, fp8_bwd and mxfp8 full-size tests
# of one shape draw the same inputs (seed = configuration number, the mode does
# not change them), and at the 235B shape the oracle takes about a minute.
_EXACT = {}


def exact_layer(d, seed: int, inp: dict, r):
    """(outputs, forward state) of the oracle for the inputs drawn by
    make_inputs(d, seed): outputs y, dx, dgate, dlogits, dw2, dw13, and the
    state the oracle's forward hands its backward; callers only read them."""
    from oracle import moe_oracle as orc
    key = (d.T, d.H, d.I, d.E, d.k, d.dtype, d.skew, seed)
    if key not in _EXACT:
        y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
        ref = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
        ref["y"] = y
        _EXACT[key] = (ref, st)
    return _EXACT[key]


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
