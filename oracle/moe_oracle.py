"""fp64 CPU oracle for the fused, dropless MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py do.  It shares no code with the HIP library;
the only thing both sides use is the seeded input generator (moe_inputs).

What it computes is the plain definition of the layer the pages describe,
written out in float64 with NumPy (a matmul is the only library routine used
as a step):

  * routing: every token goes to a few experts chosen by a router, top-8 of
    128 in the pages' layers (Prime Mega MoE news page, "Short" summary and
    "Why is MoE training communication bound?"; TE dropless-MoE page,
    "01 Why is MoE training harder than dense training?");
  * dispatch = local permutation of token rows into expert-contiguous order,
    then the expert computation as grouped GEMMs over the actual per-expert
    token counts, no dropping and no padding (TE dropless-MoE page,
    "02 Dropless vs capacity-based MoE", "03 Specialised optimisations",
    "Optimisation 1: Grouped GEMM");
  * the expert MLP is two linear layers with SwiGLU between them (Prime Mega
    MoE news page, "How does the fused kernel work?");
  * combine returns rows to token order and sums the expert results (TE
    dropless-MoE page, "Optimisation 2: dispatch and combine via NCCL EP");
  * the backward pass computes activation gradients from the weights and,
    independently, the weight gradients (neurobober digest, "Overlapping
    Backward Pass").

The pages print no formula.  The readings taken where they are silent:
  R1  gates: softmax over the k selected logits (= full softmax, keep top-k,
      renormalise);
  R2  top-k key is (-logit, expert id): ties go to the smaller id; slot j is
      the j-th largest;
  R3  rows inside an expert segment are in ascending flat index t*k+j
      (stable sort by expert);
  R4  W13 rows [0, I) are W1 (through SiLU), rows [I, 2I) are W3; no biases;
      SiLU(z) = z*sigmoid(z);
  R5  the gate multiplies the expert output in the combine;
  R6  gradient for the routing weights: dgate[t, j] = <dY[t], O_row>; the
      logit gradient is the softmax Jacobian of R1 applied to dgate;
  R7  MXFP8 (fp8_bwd backward, mxfp8 mode): E4M3FN elements, one E8M0 scale per 32
      consecutive elements along the GEMM's K; scale exponent X = the smallest
      integer with amax <= 448 * 2**X (clamped to [-127, 127]); element =
      round-to-nearest-even of v / 2**X, saturating at 448; blocks along the
      token dimension start at each expert's first row and the segment tail is
      zero-padded (TE dropless-MoE page, "03 Specialised optimisations":
      group-aware MXFP8 quantisation and MXFP8 grouped GEMM).
  R12 mxfp8 mode (Prime Mega MoE news page, "How does the fused kernel
      work?": BF16 and MXFP8 precisions): the forward GEMMs take MXFP8
      operands quantised along their K (x and W13 along H, A and W2 along I);
      SwiGLU and the combine stay in full precision; the backward is the
      fp8_bwd backward applied to this forward's state.
  R13 router projection (TE dropless-MoE page, "01 Why is MoE training
      harder than dense training?": the router is a trained component, so it
      has a gradient): logits = x W_r^T with W_r [E, H], no bias; its backward
      adds dlogits W_r to dx and gives dW_r = dlogits^T x.

Every function below is pinned by tests/test_oracle_*.py against something
other than itself (finite differences, closed forms, brute force, the
dense-FFN special case, the format definition).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Routing", "route", "silu", "sigmoid", "expert_forward", "expert_backward",
    "forward", "backward", "router_backward", "forward_with_gates",
    "e4m3fn_decode_table", "e4m3fn_encode", "e4m3fn_round", "mx_scale_exponent", "mx_quant_dequant", "mx_dequant",
    "mx_quant_dequant_tokens", "expert_backward_mxfp8", "backward_mxfp8", "expert_forward_mxfp8",
    "forward_mxfp8",
]


# --------------------------------------------------------------------------
# Routing (R1-R3)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Routing:
    idx: np.ndarray             # [T, k] int32, expert of slot j of token t
    gate: np.ndarray            # [T, k] float64
    counts: np.ndarray          # [E] int64
    offsets: np.ndarray         # [E+1] int64
    sorted_to_flat: np.ndarray  # [T*k] int64: row r of the expert-sorted order -> t*k+j
    flat_to_sorted: np.ndarray  # [T*k] int64: inverse permutation
    k: int
    E: int


def route(logits: np.ndarray, k: int) -> Routing:
    """Top-k routing with renormalised softmax gates (R1, R2) and the stable
    expert-major permutation (R3)."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    assert 1 <= k <= E
    assert np.all(np.isfinite(L)), "non-finite logits are outside the definition"
    # A stable sort of -L orders equal logits by ascending expert id: key (-L, e).
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k]
    sel = np.take_along_axis(L, idx, axis=1)
    z = np.exp(sel - sel[:, :1])
    gate = z / z.sum(axis=1, keepdims=True)
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    s2f = np.argsort(flat, kind="stable").astype(np.int64)
    f2s = np.empty_like(s2f)
    f2s[s2f] = np.arange(flat.size, dtype=np.int64)
    return Routing(idx=idx.astype(np.int32), gate=gate, counts=counts, offsets=offsets,
                   sorted_to_flat=s2f, flat_to_sorted=f2s, k=k, E=E)


# --------------------------------------------------------------------------
# Expert MLP (R4)
# --------------------------------------------------------------------------
def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    return z * sigmoid(z)


def expert_forward(xrows: np.ndarray, w13e: np.ndarray, w2e: np.ndarray) -> dict:
    """One expert on a set of token rows: G = X W13^T, A = SiLU(G1) * G3, O = A W2^T."""
    X = np.asarray(xrows, dtype=np.float64)
    W13 = np.asarray(w13e, dtype=np.float64)
    W2 = np.asarray(w2e, dtype=np.float64)
    I = W13.shape[0] // 2
    G = X @ W13.T
    G1, G3 = G[:, :I], G[:, I:]
    A = silu(G1) * G3
    O = A @ W2.T
    return {"G1": G1, "G3": G3, "A": A, "O": O}


def expert_backward(dO: np.ndarray, xrows: np.ndarray, w13e: np.ndarray, w2e: np.ndarray,
                    fwd: dict) -> dict:
    """Gradients of one expert given dL/dO for its rows.

    dA = dO W2, dW2 = dO^T A, dSwiGLU, dX = dG W13, dW13 = dG^T X.
    """
    dO = np.asarray(dO, dtype=np.float64)
    X = np.asarray(xrows, dtype=np.float64)
    W13 = np.asarray(w13e, dtype=np.float64)
    W2 = np.asarray(w2e, dtype=np.float64)
    G1, G3, A = fwd["G1"], fwd["G3"], fwd["A"]
    dA = dO @ W2
    dW2 = dO.T @ A
    s = sigmoid(G1)
    dG1 = dA * G3 * s * (1.0 + G1 * (1.0 - s))   # d/dz SiLU(z) = s (1 + z (1 - s))
    dG3 = dA * G1 * s
    dG = np.concatenate([dG1, dG3], axis=1)
    dX = dG @ W13
    dW13 = dG.T @ X
    return {"dA": dA, "dG": dG, "dX": dX, "dW13": dW13, "dW2": dW2}


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def _for_each_expert(r: Routing, body, workers: int = 1):
    """body(e, a, b) for every non-empty expert segment [a, b).  The bodies
    write disjoint rows and experts, so running them on `workers` threads
    (numpy releases the GIL in its kernels) gives the same arrays."""
    segs = [(e, a, b) for e, a, b in _segments(r) if b > a]
    if workers <= 1:
        for seg in segs:
            body(*seg)
        return
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(body, *seg) for seg in segs]:
            f.result()


def _segments(r: Routing):
    for e in range(r.E):
        a, b = int(r.offsets[e]), int(r.offsets[e + 1])
        yield e, a, b


def forward_with_gates(x, w13, w2, idx, gate):
    """Layer forward for given routing indices and (independent) gate values.

    Used for finite differences with respect to the gates."""
    idx = np.asarray(idx)
    T, k = idx.shape
    E = w13.shape[0]
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    s2f = np.argsort(flat, kind="stable")
    f2s = np.empty_like(s2f)
    f2s[s2f] = np.arange(flat.size)
    r = Routing(idx=idx, gate=np.asarray(gate, dtype=np.float64), counts=counts,
                offsets=offsets, sorted_to_flat=s2f, flat_to_sorted=f2s, k=k, E=E)
    return forward(x, w13, w2, r)


def forward(x, w13, w2, r: Routing, *, workers: int = 1):
    """Y[t] = sum_j gate[t,j] * FFN_{idx[t,j]}(x[t]) through the permuted layout.

    Returns (Y [T,H] float64, state) where state keeps what the backward needs.
    workers > 1 runs the independent experts on that many threads (same result).
    """
    return _layer_forward(x, w13, w2, r, expert_forward, workers)


def _layer_forward(x, w13, w2, r: Routing, expert_fn, workers: int = 1):
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    k = r.k
    M = T * k
    I = w13.shape[1] // 2
    tok = r.sorted_to_flat // k                    # token of each sorted row
    O = np.zeros((M, H))
    G1 = np.zeros((M, I))
    G3 = np.zeros((M, I))
    A = np.zeros((M, I))
    def one(e, a, b):
        f = expert_fn(x[tok[a:b]], w13[e], w2[e])
        O[a:b], G1[a:b], G3[a:b], A[a:b] = f["O"], f["G1"], f["G3"], f["A"]

    _for_each_expert(r, one, workers)
    # combine: gather each token's k rows back in slot order, weight by its gates
    Orows = O[r.flat_to_sorted].reshape(T, k, H)
    Y = np.einsum("tk,tkh->th", r.gate, Orows)
    return Y, {"O": O, "G1": G1, "G3": G3, "A": A}


def router_backward(gate: np.ndarray, dgate: np.ndarray, idx: np.ndarray, E: int) -> np.ndarray:
    """dL/dlogits through the renormalised top-k softmax (R1); zero off the top-k set."""
    g = np.asarray(gate, dtype=np.float64)
    dg = np.asarray(dgate, dtype=np.float64)
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dsel = g * (dg - inner)
    T = g.shape[0]
    dL = np.zeros((T, E))
    np.put_along_axis(dL, np.asarray(idx, dtype=np.int64), dsel, axis=1)
    return dL


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Router projection (R13): logits[t, e] = <x[t], W_r[e]>."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def router_projection_backward(dlogits: np.ndarray, x: np.ndarray, w_router: np.ndarray) -> dict:
    """Backward of logits = x W_r^T (R13): the router's share of dx and the
    router weight gradient."""
    dl = np.asarray(dlogits, dtype=np.float64)
    return {"dx": dl @ np.asarray(w_router, dtype=np.float64),
            "dw_router": dl.T @ np.asarray(x, dtype=np.float64)}


def backward(dy, x, w13, w2, r: Routing, state: dict, *, want_dw=True, workers: int = 1):
    """Gradients of <dY, Y> with respect to x, W13, W2, the gates and the logits
    (workers > 1: the independent experts on that many threads, same result)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    k = r.k
    M = T * k
    E = r.E
    tok = r.sorted_to_flat // k
    g_sorted = r.gate.reshape(-1)[r.sorted_to_flat]     # gate of each sorted row
    # combine backward
    dO = g_sorted[:, None] * dy[tok]
    Orows = state["O"][r.flat_to_sorted].reshape(T, k, H)
    dgate = np.einsum("th,tkh->tk", dy, Orows)
    dXp = np.zeros((M, H))
    dW13 = np.zeros(w13.shape) if want_dw else None
    dW2 = np.zeros(w2.shape) if want_dw else None
    def one(e, a, b):           # an expert with no rows keeps zero weight gradients
        fwd = {"G1": state["G1"][a:b], "G3": state["G3"][a:b], "A": state["A"][a:b]}
        g = expert_backward(dO[a:b], x[tok[a:b]], w13[e], w2[e], fwd)
        dXp[a:b] = g["dX"]
        if want_dw:
            dW13[e], dW2[e] = g["dW13"], g["dW2"]

    _for_each_expert(r, one, workers)
    # unpermute + sum over the k slots
    dX = dXp[r.flat_to_sorted].reshape(T, k, H).sum(axis=1)
    dlogits = router_backward(r.gate, dgate, r.idx, E)
    return {"dx": dX, "dw13": dW13, "dw2": dW2, "dgate": dgate, "dlogits": dlogits}


# --------------------------------------------------------------------------
# MXFP8 emulation (R7)
# --------------------------------------------------------------------------
def e4m3fn_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (sign | 4-bit exponent, bias 7 |
    3-bit mantissa; exponent field 0 is subnormal; S.1111.111 is NaN; no inf)."""
    out = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ef = (c >> 3) & 0xF
        mf = c & 0x7
        if ef == 0xF and mf == 0x7:
            out[c] = np.nan
        elif ef == 0:
            out[c] = s * (mf / 8.0) * 2.0 ** (1 - 7)
        else:
            out[c] = s * (1.0 + mf / 8.0) * 2.0 ** (ef - 7)
    return out


_E4M3_TABLE = e4m3fn_decode_table()
_E4M3_POS = _E4M3_TABLE[:0x7F]                  # codes 0..126: the finite non-negative values


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3FN value (ties to the even code), saturating at
    +-448.  Returns uint8 codes."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    # nearest grid point among the 127 non-negative finite values (ascending)
    hi = np.searchsorted(_E4M3_POS, a, side="left")         # first value >= a
    hi = np.minimum(hi, _E4M3_POS.size - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)
    # the sign bit is kept, also for values that round to zero
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def e4m3fn_round(v: np.ndarray) -> np.ndarray:
    """Value of e4m3fn_encode(v) (float64, sign kept also for zero), computed
    without building codes.

    Inside a binade [2**e, 2**(e+1)) with e >= -6 the E4M3FN magnitudes are
    the multiples of 2**(e-3) (mantissa 1.mmm); below 2**-6 (the subnormals)
    they are the multiples of 2**-9.  Consecutive codes are consecutive
    multiples and a code's last mantissa bit is the parity of its multiple, so
    rounding |v| to the nearest multiple of its binade's step with ties to the
    even multiple (numpy's round) is rounding to the nearest code with ties to
    the even code; |v| is first clipped to 448 (saturation), itself a multiple
    of its step.  frexp gives the binade exactly; every scaling is by a power
    of two, hence exact."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    _, ex = np.frexp(a)                         # a = m * 2**ex, m in [0.5, 1): binade e = ex - 1
    step = np.exp2((np.maximum(ex, -5) - 4).astype(np.float64))   # 2**(max(e, -6) - 3)
    r = np.round(a / step) * step
    return np.copysign(r, v)


def mx_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer X in [-127, 127] with amax <= 448 * 2**X (amax = 0 -> -127).

    The comparisons with 448 * 2**X are exact in float64."""
    amax = np.asarray(amax, dtype=np.float64)
    X = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    a = amax[nz]
    with np.errstate(divide="ignore"):
        x = np.ceil(np.log2(a / 448.0)).astype(np.int64)
    x = np.where(a > 448.0 * np.exp2(x.astype(np.float64)), x + 1, x)
    x = np.where(a <= 448.0 * np.exp2((x - 1).astype(np.float64)), x - 1, x)
    X[nz] = np.clip(x, -127, 127)
    return X


def mx_quant_dequant(a: np.ndarray, axis: int = -1):
    """Quantise along `axis` in blocks of 32 (length must be a multiple of 32).

    Returns (dequantised float64 array, codes uint8, scale exponents int64)."""
    a = np.asarray(a, dtype=np.float64)
    a_m = np.moveaxis(a, axis, -1)
    n = a_m.shape[-1]
    assert n % 32 == 0
    blk = a_m.reshape(a_m.shape[:-1] + (n // 32, 32))
    X = mx_scale_exponent(np.max(np.abs(blk), axis=-1))
    scaled = blk / np.exp2(X.astype(np.float64))[..., None]
    codes = e4m3fn_encode(scaled)
    deq = _E4M3_TABLE[codes] * np.exp2(X.astype(np.float64))[..., None]
    deq = np.moveaxis(deq.reshape(a_m.shape), -1, axis)
    codes = np.moveaxis(codes.reshape(a_m.shape), -1, axis)
    return deq, codes, X


def mx_dequant(a: np.ndarray, axis: int = -1) -> np.ndarray:
    """dequant(quant(a)) along `axis` in blocks of 32: the first value
    mx_quant_dequant returns, with the elements rounded by e4m3fn_round (the
    same values, without the codes)."""
    a = np.asarray(a, dtype=np.float64)
    a_m = np.moveaxis(a, axis, -1)
    n = a_m.shape[-1]
    assert n % 32 == 0
    blk = a_m.reshape(a_m.shape[:-1] + (n // 32, 32))
    scale = np.exp2(mx_scale_exponent(np.max(np.abs(blk), axis=-1)).astype(np.float64))[..., None]
    deq = e4m3fn_round(blk / scale) * scale
    return np.moveaxis(deq.reshape(a_m.shape), -1, axis)


def mx_quant_dequant_tokens(a: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Group-aware quantisation along the row (token) axis of a [M, N] array:
    32-row blocks start at each expert's first row; the tail is zero-padded."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        n = hi - lo
        npad = (n + 31) // 32 * 32
        seg = np.zeros((npad, a.shape[1]))
        seg[:n] = a[lo:hi]
        out[lo:hi] = mx_dequant(seg, axis=0)[:n]
    return out


def expert_backward_mxfp8(dYp, Xp, g, w13e, w2e, fwd: dict) -> dict:
    """One expert's share of the fp8_bwd backward (R7): the rows of one expert
    segment, every backward GEMM operand replaced by dequant(quant(.)) along
    that GEMM's K.  The gate is applied after the dgrad GEMM of W2 and folded
    into A for the W2 weight gradient.

      dA'  = Q_H(dYp) Q_H(W2[e])            (K = H)
      dXp  = Q_2I(dG) Q_2I(W13[e])          (K = 2I)
      dW2  = Q_tok(dYp)^T Q_tok(g A)        (K = tokens of e)
      dW13 = Q_tok(dG)^T Q_tok(Xp)          (K = tokens of e)

    dgate and the SwiGLU derivative use the unquantised forward state `fwd`
    (G1, G3, A of these rows).  Row-wise quantisation (along H or 2I) treats
    every row on its own; the token blocks start at the segment's first row."""
    dYp = np.asarray(dYp, dtype=np.float64)
    Xp = np.asarray(Xp, dtype=np.float64)
    n = dYp.shape[0]
    seg = np.array([0, n])
    qW2 = mx_dequant(np.asarray(w2e, dtype=np.float64), axis=0)      # [H, I], K = H
    qdYp = mx_dequant(dYp, axis=1)
    dAp = qdYp @ qW2
    A, G1, G3 = fwd["A"], fwd["G1"], fwd["G3"]
    dgate = np.sum(dAp * A, axis=1)
    dA = g[:, None] * dAp
    s = sigmoid(G1)
    dG = np.concatenate([dA * G3 * s * (1.0 + G1 * (1.0 - s)), dA * G1 * s], axis=1)
    qW13 = mx_dequant(np.asarray(w13e, dtype=np.float64), axis=0)   # [2I, H], K = 2I
    qdG = mx_dequant(dG, axis=1)
    dXp = qdG @ qW13
    dW2 = mx_quant_dequant_tokens(dYp, seg).T @ mx_quant_dequant_tokens(g[:, None] * A, seg)
    dW13 = mx_quant_dequant_tokens(dG, seg).T @ mx_quant_dequant_tokens(Xp, seg)
    return {"dXp": dXp, "dgate": dgate, "dG": dG, "dW2": dW2, "dW13": dW13}


def backward_mxfp8(dy, x, w13, w2, r: Routing, state: dict, *, workers: int = 1):
    """fp8_bwd backward of the whole layer: expert_backward_mxfp8 on every
    expert segment, then the unpermute-reduce of dX and the router backward
    exactly as in backward() (workers > 1: experts on that many threads)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    k, E = r.k, r.E
    M = T * k
    tok = r.sorted_to_flat // k
    g_sorted = r.gate.reshape(-1)[r.sorted_to_flat]
    dXp = np.zeros((M, H))
    dW13 = np.zeros(w13.shape)
    dW2 = np.zeros(w2.shape)
    dgate_sorted = np.zeros(M)
    def one(e, a, b):
        fwd = {key: state[key][a:b] for key in ("A", "G1", "G3")}
        out = expert_backward_mxfp8(dy[tok[a:b]], x[tok[a:b]], g_sorted[a:b], w13[e], w2[e], fwd)
        dXp[a:b] = out["dXp"]
        dgate_sorted[a:b] = out["dgate"]
        dW2[e] = out["dW2"]
        dW13[e] = out["dW13"]

    _for_each_expert(r, one, workers)
    dX = dXp[r.flat_to_sorted].reshape(T, k, H).sum(axis=1)
    dgate = dgate_sorted[r.flat_to_sorted].reshape(T, k)
    dlogits = router_backward(r.gate, dgate, r.idx, E)
    return {"dx": dX, "dw13": dW13, "dw2": dW2, "dgate": dgate, "dlogits": dlogits}


def expert_forward_mxfp8(xrows, w13e, w2e) -> dict:
    """One expert's forward in the mxfp8 mode (R12): both GEMMs take MXFP8
    operands, each quantised along that GEMM's K:
      G13 = Q_H(X) Q_H(W13[e])^T,  A = SiLU(G1) * G3,  O = Q_I(A) Q_I(W2[e])^T
    (W13[e] is [2I, H] and W2[e] is [H, I]: K is their last axis)."""
    X = np.asarray(xrows, dtype=np.float64)
    W13 = np.asarray(w13e, dtype=np.float64)
    W2 = np.asarray(w2e, dtype=np.float64)
    I = W13.shape[0] // 2
    G = mx_dequant(X, axis=1) @ mx_dequant(W13, axis=1).T
    G1, G3 = G[:, :I], G[:, I:]
    A = silu(G1) * G3
    O = mx_dequant(A, axis=1) @ mx_dequant(W2, axis=1).T
    return {"G1": G1, "G3": G3, "A": A, "O": O}


def forward_mxfp8(x, w13, w2, r: Routing, *, workers: int = 1):
    """Layer forward of the mxfp8 mode: forward() with expert_forward_mxfp8.
    Its backward is backward_mxfp8 applied to the state returned here."""
    return _layer_forward(x, w13, w2, r, expert_forward_mxfp8, workers)
