"""Benchmark of the MoE expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--cpu-tokens 16384] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input:
route + forward + backward of the layer (Qwen3-30B-A3B expert shape by
default: T=16384, H=2048, I=768, E=128, top-8, bf16).  Inputs are resident in
HBM before the timed region.  Prints one JSON line.

value = algorithmic GEMM FLOPs of forward + backward (18*M*H*I, M = T*k)
divided by the step time, in TFLOP/s.  Per-kernel durations come from HIP
events recorded between the library's kernels over the timed steps.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd ms & TFLOPS, Qwen3-30B-A3B shape T=16384; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (MXFP8 operands)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

FWD_KERNELS = ["tile_table", "gemm1_swiglu", "gemm2", "combine"]
FWD_KERNELS_MX8 = ["tile_table", "quant_x", "quant_w13", "gemm1_swiglu", "quant_w2", "gemm2", "combine"]
BWD_KERNELS = ["tile_table_b", "dgrad2_dswiglu", "dgrad1", "unpermute_reduce", "router_bwd", "wgrad2", "wgrad1",
               "wgrad_reduce"]
BWD_KERNELS_FP8 = ["tile_table_b", "pad_offsets", "quant_w2t", "quant_dy", "dgrad2_dswiglu", "quant_w13t",
                   "dgrad1", "unpermute_reduce", "router_bwd", "quant_dyt", "wgrad2", "quant_xt", "wgrad1",
                   "wgrad_reduce"]
# mxfp8 mode: the forward quantises each weight both ways, the backward reuses W2^T and W13^T codes
BWD_KERNELS_MXFP8 = [n for n in BWD_KERNELS_FP8 if n not in ("quant_w2t", "quant_w13t")]


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            arr[i] = h
        return arr

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def gemm_flops(d):
    MHI = d.M * d.H * d.I
    return {"gemm1_swiglu": 4 * MHI, "gemm2": 2 * MHI, "dgrad2_dswiglu": 2 * MHI, "dgrad1": 4 * MHI,
            "wgrad2": 2 * MHI, "wgrad1": 4 * MHI}


def hbm_bytes(d):
    """Algorithmic HBM bytes of the memory-bound kernels (bf16 inputs, fp8
    codes + one scale byte per 32 codes)."""
    rows = d.M * d.H * 2 + d.T * d.H * 2
    q = lambda n: n * 2 + n + n // 32            # read bf16, write codes + scales
    q2 = lambda n: n * 2 + 2 * (n + n // 32)     # read bf16, write both layouts (mxfp8 weights)
    H, I, E, M, T = d.H, d.I, d.E, d.M, d.T
    return {"combine": rows + d.M * 8, "unpermute_reduce": rows + d.M * 4,
            "quant_w2t": q(E * H * I), "quant_w13t": q(E * 2 * I * H), "quant_dy": q(T * H),
            "quant_dyt": q(M * H), "quant_xt": q(M * H), "quant_x": q(T * H),
            "quant_w13": q2(E * 2 * I * H), "quant_w2": q2(E * H * I)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_binary_hash() -> str:
    """sha256 of the built library (its device code included): recorded
    counter figures apply only to the binary they were taken on."""
    import grouped_gemm_layer_amd as gl
    h = hashlib.sha256()
    with open(gl.lib_path(), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(config: int, kernel: str):
    """HBM bytes per launch of `kernel` from the committed PMC figures
    (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or None when
    they are missing or were taken on another build of the library."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("library_sha256") != kernel_binary_hash() or rec.get("config") != config:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


def time_router_projection(g, layer, d, x, seed, K, W):
    """moe_route_project (logits GEMM + routing) and moe_router_backward on
    the layer's shape, after the timed steps (not part of a step)."""
    import numpy as np
    import torch
    rng = np.random.default_rng(seed + 1000)
    wr = torch.from_numpy(rng.standard_normal((d.E, d.H)).astype(np.float32) * 0.05).to("cuda", torch.bfloat16)
    dwr = torch.empty((d.E, d.H), dtype=torch.float32, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for _ in range(W):
        layer.route_project(x, wr)
        layer.router_backward(x, wr, dwr)
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        layer.route_project(x, wr)
        ev[i][1].record()
        layer.router_backward(x, wr, dwr)
        ev[i][2].record()
    torch.cuda.synchronize()
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    return {"project_and_route_ms": round(fwd, 4), "backward_ms": round(bwd, 4),
            "logits_flop": 2 * d.T * d.E * d.H,
            "note": "logits = x W_r^T + routing; backward: dx += dlogits W_r, dW_r = dlogits^T x"}


def time_call(fn, K, W):
    """Mean event time of fn() over K calls after W untimed ones (current stream)."""
    import numpy as np
    import torch
    for _ in range(W):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return round(float(np.mean([e[0].elapsed_time(e[1]) for e in ev])), 4)


def time_backward_accumulate(layer, dy, x, w13, w2, K, W):
    """moe_backward_accumulate (weight gradients added into the fp32 buffers)
    on the same batch, after the timed steps (not part of a step)."""
    import numpy as np
    import torch
    for _ in range(W):
        layer.backward(dy, x, w13, w2, accumulate=True)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        layer.backward(dy, x, w13, w2, accumulate=True)
        ev[i][1].record()
    torch.cuda.synchronize()
    return round(float(np.mean([e[0].elapsed_time(e[1]) for e in ev])), 4)


def vendor_ceiling(d, reps: int = 20):
    """hipBLASLt (through torch) on the layer's per-expert GEMM shapes, as a
    measured context for the MFMA roofline: the same expert shapes as batched
    products with uniform rows per expert (no gather, no fused epilogue, bf16
    output), the same flops as one dense product, and a large square product.
    Not part of a step; the layer never calls these."""
    import torch
    m = d.M // d.E
    dt = torch.bfloat16
    gen = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda *s: torch.randn(*s, device="cuda", dtype=dt, generator=gen)

    def timed(fn, flop):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        return {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}

    out = {}
    xb, w13b = rnd(d.E, m, d.H), rnd(d.E, d.H, 2 * d.I)      # right operands contiguous (K-outer)
    out["bmm_gemm1_shape"] = timed(lambda: torch.bmm(xb, w13b), 2.0 * d.E * m * d.H * 2 * d.I)
    del xb, w13b
    ab, w2b = rnd(d.E, m, d.I), rnd(d.E, d.I, d.H)
    out["bmm_gemm2_shape"] = timed(lambda: torch.bmm(ab, w2b), 2.0 * d.E * m * d.I * d.H)
    del ab, w2b
    xd, wd = rnd(d.E * m, d.H), rnd(2 * d.I, d.H)
    out["mm_gemm1_flops_dense_nt"] = timed(lambda: xd @ wd.t(), 2.0 * d.E * m * d.H * 2 * d.I)
    del xd, wd
    n = 8192
    xs, ws = rnd(n, n), rnd(n, n)
    out["mm_square_8192_nt"] = timed(lambda: xs @ ws.t(), 2.0 * n ** 3)
    del xs, ws
    out["note"] = ("hipBLASLt via torch, bf16 in and out, fp32 accumulate; batched shapes use "
                   f"{m} rows per expert; context for the practical MFMA ceiling, not part of the layer")
    return out


def copy_calibration(mib: int):
    """One plain device-to-device copy of `mib` MiB (bytes known exactly), for
    scaling the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {n} bytes read, {n} bytes written", file=sys.stderr, flush=True)
    del src, dst


def cpu_info():
    """CPU model (from /proc/cpuinfo) and the BLAS library numpy calls, with
    the threads it uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
            threads = max(int(i.get("num_threads", 0)) for i in libs)
    except Exception:
        pass
    return model, blas, threads


def cpu_baseline(d, inp, n_tokens):
    """The fp64 oracle on the first n_tokens tokens of the same batch (all
    experts, same weights): route, forward and backward timed separately."""
    from oracle import moe_oracle as orc
    model, blas, cores = cpu_info()
    n = min(n_tokens, d.T)
    x, L, dy = inp["x"][:n], inp["logits"][:n], inp["dy"][:n]
    t0 = time.perf_counter()
    r = orc.route(L, d.k)
    t1 = time.perf_counter()
    Y, st = orc.forward(x, inp["w13"], inp["w2"], r)
    t2 = time.perf_counter()
    orc.backward(dy, x, inp["w13"], inp["w2"], r, st)
    t3 = time.perf_counter()
    dt = t3 - t0
    flops = 18.0 * n * d.k * d.H * d.I
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "route_s": round(t1 - t0, 3), "forward_s": round(t2 - t1, 3), "backward_s": round(t3 - t2, 3),
            "cpu_model": model, "blas": blas,
            "sample": f"fp64 NumPy oracle, route+forward+backward of the first {n} of {d.T} tokens "
                      f"(all {d.E} experts, same weights), {dt:.2f} s wall"}


def kernel_names(mode):
    fp8_bwd = mode in ("fp8_bwd", "mxfp8")
    fp8_fwd = mode == "mxfp8"
    fwd_names = FWD_KERNELS_MX8 if fp8_fwd else FWD_KERNELS
    bwd_names = BWD_KERNELS_MXFP8 if fp8_fwd else BWD_KERNELS_FP8 if fp8_bwd else BWD_KERNELS
    fp8_gemms = (("gemm1_swiglu", "gemm2") if fp8_fwd else ()) + \
        (("dgrad2_dswiglu", "dgrad1", "wgrad2", "wgrad1") if fp8_bwd else ())
    peak = {n: (PEAK_FP8_TFLOPS if n in fp8_gemms else PEAK_BF16_TFLOPS) for n in fwd_names + bwd_names}
    return fwd_names, bwd_names, peak


def time_steps(g, layer, d, x, w13, w2, dy, logits, K, W, ev):
    """W untimed steps, then K timed ones (route + forward + backward), the
    whole region bracketed by device synchronisations; per-kernel durations
    from the events the library records between its kernels."""
    import numpy as np
    import torch
    fwd_names, bwd_names, peak = kernel_names(d.run_mode)
    nf, nb = g.num_kernels(layer.dims, "forward"), g.num_kernels(layer.dims, "backward")
    assert nf == len(fwd_names) and nb == len(bwd_names)
    fev = [ev.create(nf + 1) for _ in range(K)]
    bev = [ev.create(nb + 1) for _ in range(K)]
    rstart = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    rend = [torch.cuda.Event(enable_timing=True) for _ in range(K)]

    def step(i=None):
        if i is None:
            layer.route(logits)
            layer.forward(x, w13, w2)
            layer.backward(dy, x, w13, w2)
        else:
            rstart[i].record()
            layer.route(logits)
            rend[i].record()
            layer.forward(x, w13, w2, events=fev[i])
            layer.backward(dy, x, w13, w2, events=bev[i])

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    names = fwd_names + bwd_names
    per = {n: [] for n in names}
    fwd_ms, bwd_ms, route_ms = [], [], []
    for i in range(K):
        for j in range(nf):
            per[fwd_names[j]].append(ev.elapsed(fev[i][j], fev[i][j + 1]))
        for j in range(nb):
            per[bwd_names[j]].append(ev.elapsed(bev[i][j], bev[i][j + 1]))
        fwd_ms.append(ev.elapsed(fev[i][0], fev[i][nf]))
        bwd_ms.append(ev.elapsed(bev[i][0], bev[i][nb]))
        route_ms.append(rstart[i].elapsed_time(rend[i]))
    avg = {n: float(np.mean(v)) for n, v in per.items()}
    flops = gemm_flops(d)
    hbm = hbm_bytes(d)
    kernels = {}
    for n in names:
        ent = {"ms": round(avg[n], 4)}
        if n in flops:
            tf = flops[n] / (avg[n] * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), mfma_frac=round(tf / peak[n], 4))
        if n in hbm:
            gbs = hbm[n] / (avg[n] * 1e-3) / 1e9
            ent.update(gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        kernels[n] = ent
    total_flops = 18.0 * d.M * d.H * d.I
    gemm_ms = sum(avg[n] for n in flops)
    fwd, bwd, rte = float(np.mean(fwd_ms)), float(np.mean(bwd_ms)), float(np.mean(route_ms))
    return {
        "ms_per_step": ms_per_step, "value": total_flops / (ms_per_step * 1e-3) / 1e12,
        "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4), "route_ms": round(rte, 4),
        # the pages' "full layer" timing recomputes the forward (activation checkpointing)
        "ms_2f_plus_b": round(2.0 * fwd + bwd + rte, 4),
        "fwd_tflops": round(6.0 * d.M * d.H * d.I / (fwd * 1e-3) / 1e12, 1),
        "bwd_tflops": round(12.0 * d.M * d.H * d.I / (bwd * 1e-3) / 1e12, 1),
        "gemm_tflops": round(total_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_mfma_frac": round(sum(flops[n] / (peak[n] * 1e12) for n in flops) / (gemm_ms * 1e-3), 4),
        "kernels": kernels, "_avg": avg, "_peak": peak, "_flops": flops,
    }


# Extra workloads timed after the headline (compact figures): the skewed
# routing, the Qwen3-235B-A22B shape, the fp8_bwd mode and the mxfp8 mode.
EXTRA_WORKLOADS = [(3, None), (4, None), (5, None), (2, "mxfp8")]


def time_extra(g, mi, cfg, mode, base, K, W, ev):
    """Steps of one extra workload, with its own seeded inputs (seed = the
    configuration number); the 30B-shape workloads reuse the headline's
    device tensors of the same recipe where only the seed would differ, except
    the logits, which carry the routing."""
    import dataclasses
    import torch
    d = mi.CONFIGS[cfg]
    name = mi.CONFIG_NAMES[cfg]
    if mode is not None:
        d = dataclasses.replace(d, mode=mode)
        name += f", {mode} mode"
    print(f"[bench] extra: config {cfg}{'' if mode is None else ' ' + mode}: {name}", file=sys.stderr, flush=True)
    same_shape = (d.T, d.H, d.I, d.E, d.k) == tuple(base["dims"])
    inp = mi.make_inputs(d, cfg, want=("logits",) if same_shape else ("x", "w13", "w2", "logits", "dy"))
    dev = lambda a, dt: torch.from_numpy(a).to(device="cuda", dtype=dt)
    if same_shape:
        x, w13, w2, dy = base["x"], base["w13"], base["w2"], base["dy"]
        note = "x, W13, W2, dY: the headline's tensors (same recipe, seed 2); logits of this configuration"
    else:
        x, w13, w2, dy = (dev(inp[k], torch.bfloat16) for k in ("x", "w13", "w2", "dy"))
        note = f"inputs of this configuration (seed {cfg})"
    logits = dev(inp["logits"], torch.float32)
    del inp
    layer = g.MoeLayer(d.T, d.H, d.I, d.E, d.k, mode=d.run_mode)
    res = time_steps(g, layer, d, x, w13, w2, dy, logits, K, W, ev)
    counts = layer.routing.counts.cpu()
    out = {"workload": name, "mode": d.run_mode, "T": d.T, "H": d.H, "I": d.I, "E": d.E, "k": d.k,
           "ms_per_step": round(res["ms_per_step"], 4), "tflops": round(res["value"], 1),
           "fwd_ms": res["fwd_ms"], "bwd_ms": res["bwd_ms"], "route_ms": res["route_ms"],
           "ms_2f_plus_b": res["ms_2f_plus_b"], "gemm_tflops": res["gemm_tflops"],
           "gemm_mfma_frac": res["gemm_mfma_frac"],
           "gemm_ms": {n: v["ms"] for n, v in res["kernels"].items() if n in res["_flops"]},
           "gemm_frac": {n: v["mfma_frac"] for n, v in res["kernels"].items() if n in res["_flops"]},
           "routing": {"max_over_mean": round(float(counts.max()) * d.E / d.M, 2),
                       "empty_experts": int((counts == 0).sum())},
           "inputs": note}
    other = {n: v["ms"] for n, v in res["kernels"].items() if n not in res["_flops"] and v["ms"] >= 0.02}
    if other:
        out["other_kernels_ms"] = other
    if d.run_mode in ("fp8_bwd", "mxfp8"):
        # cached MXFP8 weights: quantised once per optimizer step, then every
        # forward and backward of that step (micro-batches, the checkpointing
        # recompute) reads the copies
        qw = time_call(lambda: layer.quantize_weights(w13, w2), K, W)
        fc = time_call(lambda: layer.forward_cached(x, w13, w2), K, W)
        bc = time_call(lambda: layer.backward_cached(dy, x), K, W)
        out["cached_weights"] = {"quantize_weights_ms": qw, "fwd_ms": fc, "bwd_ms": bc,
                                 "route_fwd_bwd_ms": round(res["route_ms"] + fc + bc, 4),
                                 "note": "forward and backward reading the MXFP8 weight copies made once per "
                                         "optimizer step by moe_quantize_weights (timed on its own)"}
    del layer, x, w13, w2, dy, logits
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def token_sweep(g, d, tokens, K, W):
    """Route + forward + backward of the shape (H, I, E, k) of `d` at other
    token counts, bf16, K timed steps after W untimed ones (device clock
    around the whole region).  `weight_floor_ms` is the time HBM needs for the
    weight traffic alone at 8 TB/s: every bf16 weight read by the forward and
    by the dgrad GEMMs, the fp32 weight gradients written once; below a few
    hundred rows per expert a step approaches it."""
    import torch
    H, I, E, k = d.H, d.I, d.E, d.k
    w_elems = E * 3 * H * I
    floor_ms = (2 * 2 * w_elems + 4 * w_elems) / (PEAK_HBM_GBS * 1e9) * 1e3
    out = []
    for T in tokens:
        gen = torch.Generator(device="cuda").manual_seed(T)
        bf = torch.bfloat16
        x = torch.randn(T, H, device="cuda", generator=gen).to(bf)
        w13 = (torch.randn(E, 2 * I, H, device="cuda", generator=gen) * 0.02).to(bf)
        w2 = (torch.randn(E, H, I, device="cuda", generator=gen) * 0.02).to(bf)
        logits = torch.randn(T, E, device="cuda", generator=gen)
        dy = torch.randn(T, H, device="cuda", generator=gen).to(bf)
        layer = g.MoeLayer(T, H, I, E, k, mode="bf16")

        def step():
            layer.route(logits)
            layer.forward(x, w13, w2)
            layer.backward(dy, x, w13, w2)
        for _ in range(W):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / K
        out.append({"T": T, "rows_per_expert": T * k / E, "ms_per_step": round(ms, 4),
                    "tflops": round(18.0 * T * k * H * I / ms / 1e9, 1), "weight_floor_ms": round(floor_ms, 4)})
        del layer, x, w13, w2, logits, dy
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--mode", choices=["bf16", "mxfp8", "fp8_bwd"], default=None,
                    help="run the configuration's shape in another precision mode")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip everything after the headline steps: the router projection, accumulate-into "
                         "and checkpointing timings and the other workloads (profiled runs: every GEMM launch "
                         "is then a plain step's)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads (skewed routing, 235B shape, fp8_bwd, mxfp8)")
    ap.add_argument("--extra-steps", type=int, default=10, help="timed steps per extra workload")
    ap.add_argument("--vendor-ceiling", action="store_true",
                    help="also time hipBLASLt on the per-expert GEMM shapes (roofline context)")
    ap.add_argument("--token-sweep", type=str, default="",
                    help="comma-separated token counts: also time route + forward + backward of the "
                         "configuration's shape at each (bf16 mode, seeded random inputs on the device)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain copy of this many MiB before the timed region (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              f"(this build runs on a single MI355X and has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import grouped_gemm_layer_amd as g

    d = mi.CONFIGS[args.config]
    workload = mi.CONFIG_NAMES[args.config]
    if args.mode is not None and args.mode != d.run_mode:
        import dataclasses
        d = dataclasses.replace(d, mode=args.mode)
        workload += f", {args.mode} mode"
    seed = args.config if args.seed is None else args.seed
    print(f"[bench] config {args.config}: {workload}", file=sys.stderr, flush=True)
    inp = mi.make_inputs(d, seed)
    torch.cuda.set_device(0)
    layer = g.MoeLayer(d.T, d.H, d.I, d.E, d.k, mode=d.run_mode)
    adt = layer.act_dtype
    dev = lambda a, dt: torch.from_numpy(a).to(device="cuda", dtype=dt)
    x, w13, w2, dy = dev(inp["x"], adt), dev(inp["w13"], adt), dev(inp["w2"], adt), dev(inp["dy"], adt)
    logits = dev(inp["logits"], torch.float32)
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)

    ev = HipEvents()
    K, W = args.steps, args.warmup
    res = time_steps(g, layer, d, x, w13, w2, dy, logits, K, W, ev)
    avg, peak, flops = res["_avg"], res["_peak"], res["_flops"]
    dom = max(flops, key=lambda n: avg[n])
    dom_tf = flops[dom] / (avg[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 2), "peak": peak[dom],
                "unit": "TFLOP/s", "frac": round(dom_tf / peak[dom], 4),
                "traffic": recorded_traffic(args.config, dom),
                "flops_per_launch": flops[dom], "avg_launch_ms": round(avg[dom], 4)}
    out = {
        "metric": METRIC, "value": round(res["value"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp8_bwd": "bf16 fwd + mxfp8 bwd", "mxfp8": "mxfp8"}[d.run_mode],
        "data": "synthetic",
        "config": {"workload": workload, "T": d.T, "H": d.H, "I": d.I, "E": d.E,
                   "k": d.k, "mode": d.run_mode, "seed": seed},
    }
    out.update({k: v for k, v in res.items() if not k.startswith("_") and k not in ("ms_per_step", "value")})
    out.update({"roofline": roofline, "cpu_baseline": None})
    if not args.no_extras:
        if d.run_mode != "fp32":   # the router projection (x W_r^T -> route; its backward), timed on its own
            out["router_projection"] = time_router_projection(g, layer, d, x, seed, K, W)
        # the backward with the weight gradients added into fp32 main-gradient buffers, timed on its own
        out["bwd_accumulate_ms"] = time_backward_accumulate(layer, dy, x, w13, w2, K, W)
        # activation checkpointing: route + forward keeping no state + recompute (the saved
        # state only, no y) + backward
        nosave = time_call(lambda: layer.forward(x, w13, w2, keep_saved=False), K, W)
        rec = time_call(lambda: layer.forward_recompute(x, w13, w2), K, W)
        out["fwd_nosave_ms"] = nosave
        out["fwd_recompute_ms"] = rec
        out["ms_checkpointed_step"] = round(out["route_ms"] + nosave + rec + out["bwd_ms"], 4)
    if args.vendor_ceiling:
        out["vendor_ceiling"] = vendor_ceiling(d)
    if args.token_sweep:
        layer = None
        torch.cuda.empty_cache()
        out["token_sweep"] = token_sweep(g, d, [int(v) for v in args.token_sweep.split(",")], K, W)
    if not args.no_extras and not args.no_workloads and args.config == 2 and args.mode is None:
        del layer
        torch.cuda.empty_cache()
        base = {"dims": (d.T, d.H, d.I, d.E, d.k), "x": x, "w13": w13, "w2": w2, "dy": dy}
        out["workloads"] = [time_extra(g, mi, cfg, mode, base, args.extra_steps, min(W, 3), ev)
                            for cfg, mode in EXTRA_WORKLOADS]
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, inp, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
