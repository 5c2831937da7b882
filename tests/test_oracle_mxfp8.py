"""Pins for the oracle's MXFP8 emulation: the E4M3FN decode table against
torch's float8_e4m3fn type, rounding against torch's conversion and
hand-built midpoints, the E8M0 scale rule, group-aware token blocks, and the
quantised backward against the exact one."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
import moe_inputs as mi


def test_decode_table_matches_torch_float8():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    tab = orc.e4m3fn_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert nan.sum() == 2                       # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], tab[~nan])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9


def test_representable_values_round_trip():
    tab = orc.e4m3fn_decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    enc = orc.e4m3fn_encode(tab[codes])
    assert np.array_equal(enc, codes)


def test_encode_matches_torch_conversion_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-448, 448, 20000)])
    ours = orc.e4m3fn_encode(v)
    ref = torch.tensor(v, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    zero = (orc.e4m3fn_decode_table()[ours] == 0)
    # torch and we agree on every code (zeros compared by value: +-0 both encode zero)
    assert np.array_equal(ours[~zero], ref[~zero])
    assert np.all((ref[zero] & 0x7F) == 0)


def test_round_half_to_even_midpoints():
    # between 1.0 (code 0x38, even) and 1.125 (0x39): midpoint 1.0625 -> 1.0
    # between 1.125 (0x39) and 1.25 (0x3A, even): midpoint 1.1875 -> 1.25
    # subnormal: between 0 and 2^-9: 2^-10 -> 0 ; between 2^-9 (odd) and 2^-8 (even) -> 2^-8
    v = np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, -1.0625, 464.0, 1e6, -1e6])
    enc = orc.e4m3fn_encode(v)
    assert enc.tolist() == [0x38, 0x3A, 0x00, 0x02, 0xB8, 0x7E, 0x7E, 0xFE]


def test_round_equals_decoded_encoding():
    """e4m3fn_round (the value, computed from the binade's step) equals the
    decoded code of e4m3fn_encode (nearest of the 127 table values, ties to the
    even code) on every code value, every midpoint between neighbours (and one
    ulp either side), random values over all binades, subnormals, saturation
    and signed zeros."""
    tab = orc.e4m3fn_decode_table()
    pos = tab[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2.0
    rng = np.random.default_rng(12)
    v = np.concatenate([pos, mids, np.nextafter(mids, 0.0), np.nextafter(mids, 1e9),
                        np.exp2(rng.uniform(-14, 10, 50000)), rng.uniform(0, 2.0 ** -6, 5000),
                        [0.0, 448.0, 449.0, 464.0, 479.99, 480.0, 1e9, 2.0 ** -10, 2.0 ** -11]])
    v = np.concatenate([v, -v])
    ref = np.copysign(tab[orc.e4m3fn_encode(v) & 0x7F], v)
    got = orc.e4m3fn_round(v)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(v))


def test_dequant_equals_quant_dequant():
    rng = np.random.default_rng(13)
    a = rng.standard_normal((48, 256)) * np.exp(rng.uniform(-30, 30, (48, 1)))
    a[0, :32] = 0.0
    a[1, :32] = -0.0
    a[2, 32:64] = 1.0625 * 2.0 ** np.arange(-16, 16)
    for axis in (0, 1):
        b = a if axis == 1 else a[:, :96].T.copy()
        deq, _, _ = orc.mx_quant_dequant(b, axis=axis)
        assert np.array_equal(orc.mx_dequant(b, axis=axis), deq)


def test_scale_rule():
    amax = np.array([448.0, 448.00001, 224.0, 224.0001, 1.0, 0.0, 3.5, 1e-30, 2.0 ** 130])
    X = orc.mx_scale_exponent(amax)
    assert X.tolist()[:5] == [0, 1, -1, 0, -8]
    assert X[5] == -127
    # property: amax / 2^X in (224, 448] whenever no clamp applies
    rng = np.random.default_rng(1)
    a = np.exp(rng.uniform(-40, 40, 5000))
    X = orc.mx_scale_exponent(a)
    ratio = a / np.exp2(X.astype(np.float64))
    assert np.all(ratio <= 448.0) and np.all(ratio > 224.0)
    assert X[-1] <= 127 and orc.mx_scale_exponent(np.array([2.0 ** 130]))[0] == 122


def test_block_quant_error_bound():
    """Each element is within half an E4M3 step (relative 2^-4) of its block-scaled value,
    or within the subnormal step 2^-10 * 2^X."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-5, 5, (64, 1)))
    deq, codes, X = orc.mx_quant_dequant(a, axis=1)
    scale = np.repeat(np.exp2(X.astype(np.float64)), 32, axis=1)
    err = np.abs(deq - a)
    bound = np.maximum(np.abs(a) * 2.0 ** -4, 2.0 ** -10 * scale)
    assert np.all(err <= bound * (1 + 1e-12))
    # quantising the dequantised array again is exact (idempotent)
    deq2, _, _ = orc.mx_quant_dequant(deq, axis=1)
    assert np.array_equal(deq, deq2)


def test_group_aware_token_blocks():
    rng = np.random.default_rng(3)
    offsets = np.array([0, 5, 5, 70, 100])       # segments of 5, 0, 65, 30 rows
    a = rng.standard_normal((100, 64))
    a[5:70] *= 1000.0                            # a loud segment must not change its neighbours
    q = orc.mx_quant_dequant_tokens(a, offsets)
    for lo, hi in ((0, 5), (70, 100)):
        seg = np.zeros(((hi - lo + 31) // 32 * 32, 64))
        seg[:hi - lo] = a[lo:hi]
        ref, _, _ = orc.mx_quant_dequant(seg, axis=0)
        assert np.array_equal(q[lo:hi], ref[:hi - lo])
    # rows 5..36 form one block, 37..68 the next, 69 a block of its own
    single, _, _ = orc.mx_quant_dequant(np.vstack([a[69:70], np.zeros((31, 64))]), axis=0)
    assert np.array_equal(q[69], single[0])


def test_quantised_backward_close_to_exact():
    d = mi.LayerDims(T=128, H=128, I=64, E=4, k=2, dtype="bf16", mode="fp8_bwd")
    inp = mi.make_inputs(d, 5)
    r = orc.route(inp["logits"], d.k)
    Y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    g = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    q = orc.backward_mxfp8(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    for key in ("dx", "dw13", "dw2", "dgate", "dlogits"):
        rel = np.max(np.abs(q[key] - g[key])) / np.max(np.abs(g[key]))
        assert 1e-4 < rel < 0.15, (key, rel)     # quantisation is visible but bounded


def test_quantised_backward_structure_with_identity_quantiser(monkeypatch):
    """With the quantiser replaced by the identity the fp8_bwd backward must equal
    the exact backward: this pins which operands meet in which GEMM."""
    d = mi.LayerDims(T=96, H=64, I=32, E=5, k=2, dtype="fp32")
    inp = mi.make_inputs(d, 6)
    r = orc.route(inp["logits"], d.k)
    Y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    g = orc.backward(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    monkeypatch.setattr(orc, "mx_dequant", lambda a, axis=-1: np.asarray(a, np.float64))
    monkeypatch.setattr(orc, "mx_quant_dequant_tokens", lambda a, offsets: np.asarray(a, np.float64))
    q = orc.backward_mxfp8(inp["dy"], inp["x"], inp["w13"], inp["w2"], r, st)
    for key in ("dx", "dw13", "dw2", "dgate", "dlogits"):
        rel = np.max(np.abs(q[key] - g[key])) / np.max(np.abs(g[key]))
        assert rel < 1e-12, (key, rel)


def test_quantised_operands_are_blocked_along_each_gemms_k(monkeypatch):
    """Records every quantiser call of one expert's fp8_bwd backward: each GEMM
    operand must be blocked along that GEMM's reduction dimension (H for the
    dgrad of W2, 2I for the dgrad of W13, the expert's tokens for the weight
    gradients), and the token-wise operands are dY, gate*A, dG13 and x."""
    rng = np.random.default_rng(7)
    n, H, I = 40, 64, 32
    dYp, Xp = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    g = rng.uniform(0.1, 1.0, n)
    w13e, w2e = rng.standard_normal((2 * I, H)), rng.standard_normal((H, I))
    fwd = orc.expert_forward(Xp, w13e, w2e)
    calls = []

    def rec(a, axis=-1):
        a = np.asarray(a, np.float64)
        calls.append(("rows", a.shape, axis % a.ndim))
        return a

    def rec_tok(a, offsets):
        a = np.asarray(a, np.float64)
        calls.append(("tokens", a.shape, tuple(int(o) for o in offsets), a.copy()))
        return a

    monkeypatch.setattr(orc, "mx_dequant", rec)
    monkeypatch.setattr(orc, "mx_quant_dequant_tokens", rec_tok)
    out = orc.expert_backward_mxfp8(dYp, Xp, g, w13e, w2e, fwd)
    row_calls = sorted((c[1], c[2]) for c in calls if c[0] == "rows")
    # W2 [H, I] along H (axis 0); dY [n, H] along H (axis 1); W13 [2I, H] along 2I (axis 0); dG [n, 2I] along 2I
    assert row_calls == sorted([((H, I), 0), ((n, H), 1), ((2 * I, H), 0), ((n, 2 * I), 1)])
    tok = [c for c in calls if c[0] == "tokens"]
    assert len(tok) == 4 and all(c[2] == (0, n) for c in tok)
    arrays = [c[3] for c in tok]
    expected = [dYp, g[:, None] * fwd["A"], out["dG"], Xp]
    for ref in expected:
        assert any(a.shape == ref.shape and np.array_equal(a, ref) for a in arrays)


def test_mxfp8_forward_with_identity_quantiser_is_exact(monkeypatch):
    d = mi.LayerDims(T=96, H=64, I=32, E=5, k=2, dtype="fp32")
    inp = mi.make_inputs(d, 8)
    r = orc.route(inp["logits"], d.k)
    Y, st = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    monkeypatch.setattr(orc, "mx_dequant", lambda a, axis=-1: np.asarray(a, np.float64))
    Yq, stq = orc.forward_mxfp8(inp["x"], inp["w13"], inp["w2"], r)
    assert np.max(np.abs(Yq - Y)) <= 1e-12 * np.max(np.abs(Y))
    for key in ("G1", "G3", "A", "O"):
        assert np.max(np.abs(stq[key] - st[key])) <= 1e-12 * np.max(np.abs(st[key]))


def test_mxfp8_forward_operands_blocked_along_k(monkeypatch):
    rng = np.random.default_rng(9)
    n, H, I = 24, 64, 32
    calls = []

    def rec(a, axis=-1):
        a = np.asarray(a, np.float64)
        calls.append((a.shape, axis % a.ndim))
        return a

    monkeypatch.setattr(orc, "mx_dequant", rec)
    orc.expert_forward_mxfp8(rng.standard_normal((n, H)), rng.standard_normal((2 * I, H)),
                             rng.standard_normal((H, I)))
    # x [n, H] and W13 [2I, H] along H; A [n, I] and W2 [H, I] along I
    assert sorted(calls) == sorted([((n, H), 1), ((2 * I, H), 1), ((n, I), 1), ((H, I), 1)])


def test_mxfp8_forward_exact_on_representable_operands():
    """x and W13 built from E4M3 codes times one power of two per 32-block are
    MXFP8 values already: the first GEMM (G1, G3) must equal the exact one."""
    rng = np.random.default_rng(10)
    tab = orc.e4m3fn_decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(tab[c])])

    def representable(rows, cols):
        codes = rng.choice(finite, size=(rows, cols))
        v = tab[codes]
        v[:, ::32] = 448.0 * np.sign(v[:, ::32] + 0.5)        # every block holds amax 448 * 2^X
        scale = np.exp2(rng.integers(-6, 4, size=(rows, cols // 32))).repeat(32, axis=1)
        return v * scale

    x, w13 = representable(40, 64), representable(2 * 32, 64)
    w2 = rng.standard_normal((64, 32))
    q = orc.expert_forward_mxfp8(x, w13, w2)
    e = orc.expert_forward(x, w13, w2)
    assert np.array_equal(q["G1"], e["G1"]) and np.array_equal(q["G3"], e["G3"])
    assert not np.array_equal(q["O"], e["O"])                  # A is not representable


def test_mxfp8_forward_close_to_exact():
    d = mi.LayerDims(T=128, H=128, I=64, E=4, k=2, dtype="bf16", mode="mxfp8")
    inp = mi.make_inputs(d, 11)
    r = orc.route(inp["logits"], d.k)
    Y, _ = orc.forward(inp["x"], inp["w13"], inp["w2"], r)
    Yq, _ = orc.forward_mxfp8(inp["x"], inp["w13"], inp["w2"], r)
    rel = np.max(np.abs(Yq - Y)) / np.max(np.abs(Y))
    assert 1e-4 < rel < 0.15, rel
