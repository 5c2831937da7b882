"""Seeded synthetic inputs for the MoE expert layer (shared by the GPU path's
tests/bench and by the CPU oracle's tests).

This module holds no arithmetic of the layer itself: it draws random numbers,
scales them, rounds them to the storage dtype and packs bf16 bit patterns.

The workloads follow the pages' layer benchmark: a single MoE layer with 128
experts, top-8 routing and random routing ("Prime Intellect releases Prime
Mega MoE", section "How fast is Prime Mega MoE?", the single-layer table), on
the Qwen3-30B-A3B and Qwen3-235B-A22B expert shapes at a sequence of 16384
tokens (same section, the training-step paragraph).

Recipe (per configuration, seed = configuration number unless overridden):
  np.random.SeedSequence(seed).spawn(6) children, in the order
  x, W13, W2, logits, dY, rank.  Normals are standard_normal(float32), then
  scaled: x ~ N(0,1), W13 and W2 ~ N(0, 0.02), logits ~ N(0,1), dY ~ N(0,1).
  The skewed configuration adds a per-expert logit bias
  -1.5 * ln(rank_e), rank = 1 + permutation(E) (a Zipf(s=1.2) popularity
  ranking, scaled by 1.25 so that some experts receive no token).
  bf16 workloads round every activation/weight tensor to bf16 (round to
  nearest even) on the host; logits stay fp32.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["LayerDims", "CONFIGS", "make_inputs", "bf16_round", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "config_dims"]


@dataclasses.dataclass(frozen=True)
class LayerDims:
    T: int          # tokens
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # number of experts
    k: int          # experts per token
    dtype: str      # "fp32" | "bf16" (activation / weight storage)
    skew: bool = False   # Zipf-biased router logits
    mode: str = ""       # "fp32" | "bf16" | "fp8_bwd" | "mxfp8"; default = dtype

    @property
    def M(self) -> int:
        return self.T * self.k

    @property
    def run_mode(self) -> str:
        return self.mode or self.dtype


# The five workloads (index 1..5).  Index 0 is unused so that the numbering
# matches the seed convention (seed = configuration number).
CONFIGS = {
    1: LayerDims(T=64, H=128, I=64, E=8, k=2, dtype="fp32"),
    2: LayerDims(T=16384, H=2048, I=768, E=128, k=8, dtype="bf16"),
    3: LayerDims(T=16384, H=2048, I=768, E=128, k=8, dtype="bf16", skew=True),
    4: LayerDims(T=16384, H=4096, I=1536, E=128, k=8, dtype="bf16"),
    5: LayerDims(T=16384, H=2048, I=768, E=128, k=8, dtype="bf16", mode="fp8_bwd"),
}

CONFIG_NAMES = {
    1: "tiny fp32 layer T=64 H=128 I=64 E=8 top-2",
    2: "Qwen3-30B-A3B MoE layer T=16384 H=2048 I=768 E=128 top-8 bf16",
    3: "Qwen3-30B-A3B MoE layer, Zipf-skewed routing, bf16",
    4: "Qwen3-235B-A22B MoE layer T=16384 H=4096 I=1536 E=128 top-8 bf16",
    5: "Qwen3-30B-A3B MoE layer, bf16 forward + MXFP8 backward",
}


def config_dims(n: int) -> LayerDims:
    return CONFIGS[n]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly the bf16-rounded inputs."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def _normal(ss: np.random.SeedSequence, shape, scale: float) -> np.ndarray:
    g = np.random.default_rng(ss)
    out = g.standard_normal(size=int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def make_inputs(dims: LayerDims, seed: int, *, want=("x", "w13", "w2", "logits", "dy")) -> dict:
    """Return a dict of float32 numpy arrays (bf16-valued for bf16 workloads).

    Keys: x [T,H], w13 [E,2I,H], w2 [E,H,I], logits [T,E] (always fp32 values),
    dy [T,H].  Only the keys in `want` are generated (others are skipped but the
    seed streams stay the same, so every tensor is independent of the others).
    """
    T, H, I, E = dims.T, dims.H, dims.I, dims.E
    ch = np.random.SeedSequence(seed).spawn(6)
    out = {}
    rnd = bf16_round if dims.dtype == "bf16" else (lambda a: a)
    if "x" in want:
        out["x"] = rnd(_normal(ch[0], (T, H), 1.0))
    if "w13" in want:
        out["w13"] = rnd(_normal(ch[1], (E, 2 * I, H), 0.02))
    if "w2" in want:
        out["w2"] = rnd(_normal(ch[2], (E, H, I), 0.02))
    if "logits" in want:
        lg = _normal(ch[3], (T, E), 1.0)
        if dims.skew:
            rank = 1 + np.random.default_rng(ch[5]).permutation(E)
            bias = (-1.5 * np.log(rank.astype(np.float64))).astype(np.float32)
            lg = (lg + bias[None, :]).astype(np.float32)
        out["logits"] = lg
    if "dy" in want:
        out["dy"] = rnd(_normal(ch[4], (T, H), 1.0))
    return out


def small_dims(T=300, H=256, I=128, E=8, k=2, dtype="bf16", skew=False, mode="") -> LayerDims:
    """A small shape that still spans several GEMM tiles and a ragged tail."""
    return LayerDims(T=T, H=H, I=I, E=E, k=k, dtype=dtype, skew=skew, mode=mode)
