"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe.h declares, sizes its workspaces consistently, and
rejects invalid calls with the documented status before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import grouped_gemm_layer_amd as g
    if not os.path.exists(g.lib_path()):
        pytest.fail("libmoe_gfx950.so is not built (python -m grouped_gemm_layer_amd.build_lib)")
    return g, g.load_library()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    g, lib = _lib()
    names = _declared_functions()
    assert set(names) >= {"moe_workspace_size", "moe_route", "moe_forward", "moe_backward", "moe_status_str"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    g, lib = _lib()
    for st in range(7):
        assert len(g.status_str(st)) > 0


def test_workspace_sizes_scale():
    g, lib = _lib()
    d = g.Dims.of(16384, 2048, 768, 128, 8, "bf16")
    rws, saved, fws, bws = g.workspace_size(d)
    M = 16384 * 8
    assert saved >= M * 2 * 768 * 2
    assert fws >= M * (768 + 2048) * 2
    assert bws >= M * (3 * 768 + 2048) * 2
    d32 = g.Dims.of(64, 128, 64, 8, 2, "fp32")
    assert g.workspace_size(d32)[1] >= 128 * 128 * 4


@pytest.mark.parametrize("dims,status", [
    ((0, 128, 64, 8, 2, 1), 2), ((16, 128, 64, 8, 9, 1), 2), ((16, -1, 64, 8, 2, 1), 2),
    ((16, 100, 64, 8, 2, 1), 3), ((16, 128, 96, 8, 2, 1), 3), ((16, 128, 64, 8, 2, 2), 3),
    ((16, 128, 64, 1024, 2, 1), 3), ((16, 128, 64, 64, 33, 1), 3), ((16, 128, 64, 8, 2, 7), 3),
    ((16, 192, 64, 8, 2, 3), 3), ((1 << 20, 4096, 1536, 128, 8, 1), 3),
])
def test_invalid_dims(dims, status):
    g, lib = _lib()
    d = g.Dims(*dims)
    sz = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(d), ctypes.byref(sz), None, None, None) == status


class _FakeTensor:
    """Stands for a device buffer: only its address is used (no launch happens)."""

    def __init__(self, addr, n=1 << 30):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n


def _fake_routing(g, base=0x7F0000000000):
    f = [_FakeTensor(base + i * 0x100000) for i in range(6)]
    return g.RoutingBuffers(*f)


def test_route_argument_errors_return_before_launch():
    g, lib = _lib()
    d = g.Dims.of(64, 128, 64, 8, 2, "bf16")
    r = _fake_routing(g)
    logits = _FakeTensor(0x7E0000000000)
    ws = _FakeTensor(0x7D0000000000, 16)          # too small
    with pytest.raises(g.MoeError) as ei:
        g.route(d, logits, r, ws, stream=_NullStream())
    assert ei.value.status == 5
    with pytest.raises(g.MoeError) as ei:
        g.route(d, _FakeTensor(0x7E0000000004), r, _FakeTensor(0x7D0000000000), stream=_NullStream())
    assert ei.value.status == 4                     # misaligned logits
    bad = _fake_routing(g)
    bad.gate = None
    with pytest.raises((g.MoeError, AttributeError)):
        g.route(d, logits, bad, _FakeTensor(0x7D0000000000), stream=_NullStream())
    st = lib.moe_route(ctypes.byref(d), None, None, None, 0, None)
    assert st == 1


def test_forward_backward_argument_errors():
    g, lib = _lib()
    d = g.Dims.of(64, 128, 64, 8, 2, "bf16")
    r = _fake_routing(g)
    t = lambda i: _FakeTensor(0x7C0000000000 + i * 0x1000000)
    with pytest.raises(g.MoeError) as ei:
        g.forward(d, t(0), t(1), t(2), r, t(3), t(4), _FakeTensor(0x7B0000000000, 255), stream=_NullStream())
    assert ei.value.status == 5
    with pytest.raises(g.MoeError) as ei:
        g.forward(d, t(0), None, t(2), r, t(3), t(4), t(5), stream=_NullStream())
    assert ei.value.status == 1
    with pytest.raises(g.MoeError) as ei:
        g.backward(d, t(0), t(1), t(2), t(3), r, t(4), t(5), t(6), t(7), t(8), None,
                   _FakeTensor(0x7B0000000000, 1), stream=_NullStream())
    assert ei.value.status == 5
    with pytest.raises(g.MoeError) as ei:
        g.backward(d, t(0), t(1), t(2), t(3), r, t(4), t(5), t(6), _FakeTensor(0x7C0000000010), t(8), None,
                   t(9), stream=_NullStream())
    assert ei.value.status == 4
    # accumulate-into shares the checks (errors before any launch)
    with pytest.raises(g.MoeError) as ei:
        g.backward(d, t(0), t(1), t(2), t(3), r, t(4), t(5), None, t(7), t(8), None, t(9),
                   stream=_NullStream(), accumulate=True)
    assert ei.value.status == 1
    with pytest.raises(g.MoeError) as ei:
        g.backward(d, t(0), t(1), t(2), t(3), r, t(4), t(5), t(6), t(7), t(8), None,
                   _FakeTensor(0x7B0000000000, 1), stream=_NullStream(), accumulate=True)
    assert ei.value.status == 5
    # saved may be NULL for moe_forward (nothing kept for a backward): the
    # call gets past the pointer checks to the workspace check
    with pytest.raises(g.MoeError) as ei:
        g.forward(d, t(0), t(1), t(2), r, t(3), None, _FakeTensor(0x7B0000000000, 255), stream=_NullStream())
    assert ei.value.status == 5
    # the checkpointing recompute has moe_forward's checks, without y, and needs saved
    with pytest.raises(g.MoeError) as ei:
        g.forward_recompute(d, t(0), t(1), t(2), r, None, t(5), stream=_NullStream())
    assert ei.value.status == 1
    with pytest.raises(g.MoeError) as ei:
        g.forward_recompute(d, t(0), t(1), None, r, t(4), t(5), stream=_NullStream())
    assert ei.value.status == 1
    with pytest.raises(g.MoeError) as ei:
        g.forward_recompute(d, t(0), t(1), t(2), r, t(4), _FakeTensor(0x7B0000000000, 255), stream=_NullStream())
    assert ei.value.status == 5
    with pytest.raises(g.MoeError) as ei:
        g.forward_recompute(d, _FakeTensor(0x7C0000000010), t(1), t(2), r, t(4), t(5), stream=_NullStream())
    assert ei.value.status == 4
    for dbad in (g.Dims.of(64, 128, 64, 8, 2, "mxfp8"), g.Dims.of(64, 192, 64, 8, 2, "fp8_bwd")):
        with pytest.raises(g.MoeError) as ei:
            g.forward(dbad, t(0), t(1), t(2), r, t(3), t(4), t(5), stream=_NullStream())
        assert ei.value.status == 3
        with pytest.raises(g.MoeError) as ei:
            g.forward_recompute(dbad, t(0), t(1), t(2), r, t(4), t(5), stream=_NullStream())
        assert ei.value.status == 3
        with pytest.raises(g.MoeError) as ei:
            g.backward(dbad, t(0), t(1), t(2), t(3), r, t(4), t(5), t(6), t(7), t(8), None, t(9),
                       stream=_NullStream())
        assert ei.value.status == 3


def test_num_kernels_by_mode():
    g, lib = _lib()
    bf = g.Dims.of(64, 128, 64, 8, 2, "bf16")
    f8 = g.Dims.of(64, 128, 64, 8, 2, "fp8_bwd")
    assert g.num_kernels(bf, "route") == 4 and g.num_kernels(bf, "forward") == 4
    assert g.num_kernels(bf, "backward") == 8
    assert g.num_kernels(f8, "forward") == 4 and g.num_kernels(f8, "backward") == 14
    assert lib.moe_num_kernels(ctypes.byref(g.Dims.of(0, 128, 64, 8, 2, "bf16")), 1) == -1
    assert lib.moe_num_kernels(ctypes.byref(bf), 7) == -1


def test_fp8_bwd_workspace_holds_quantised_operands():
    g, lib = _lib()
    T, H, I, E, k = 16384, 2048, 768, 128, 8
    bws_bf16 = g.workspace_size(g.Dims.of(T, H, I, E, k, "bf16"))[3]
    rws, saved, fws, bws = g.workspace_size(g.Dims.of(T, H, I, E, k, "fp8_bwd"))
    M = T * k
    Mp = g.mxfp8_grouped_capacity(M, E)
    assert Mp % 128 == 0 and Mp >= M + 127 * E
    codes = T * H + E * 3 * I * H + M * 2 * I + Mp * (2 * H + 3 * I)
    # everything of the bf16 backward except dG13 and gate*A (quantised in
    # the dgrad epilogue, never stored), plus codes and scales of every operand
    assert bws >= bws_bf16 - M * 3 * I * 2 + codes * 33 // 32
    assert saved == M * 2 * I * 4                         # G13 kept in fp32


def test_mxfp8_quantize_argument_errors():
    g, lib = _lib()
    t = lambda i: _FakeTensor(0x7C0000000000 + i * 0x1000000)
    q = lib.moe_mxfp8_quantize
    assert q(None, 64, 64, 1, t(1).addr, t(2).addr, None) == 1
    assert q(t(0).addr, 0, 64, 1, t(1).addr, t(2).addr, None) == 2
    assert q(t(0).addr, 64, 64, 2, t(1).addr, t(2).addr, None) == 2
    assert q(t(0).addr, 64, 48, 1, t(1).addr, t(2).addr, None) == 3      # cols % 32
    assert q(t(0).addr, 64, 64, 0, t(1).addr, t(2).addr, None) == 3      # rows % 128 when along = 0
    assert q(t(0).addr + 16, 64, 64, 1, t(1).addr, t(2).addr, None) == 4
    qg = lib.moe_mxfp8_quantize_grouped
    cap = g.mxfp8_grouped_capacity(100, 4)
    assert cap == 128 + 4 * 128
    assert qg(t(0).addr, 100, 64, t(1).addr, 4, cap, None, t(3).addr, t(4).addr, None) == 1
    assert qg(t(0).addr, 100, 64, t(1).addr, 4, cap - 128, t(2).addr, t(3).addr, t(4).addr, None) == 3
    assert qg(t(0).addr, 100, 64, t(1).addr, 4, cap + 32, t(2).addr, t(3).addr, t(4).addr, None) == 3
    assert qg(t(0).addr, 100, 64, t(1).addr + 4, 4, cap, t(2).addr, t(3).addr, t(4).addr, None) == 4


class _NullStream:
    cuda_stream = 0


def test_mxfp8_mode_dims_and_kernel_counts():
    g, lib = _lib()
    ok = g.Dims.of(64, 128, 128, 8, 2, "mxfp8")
    assert g.num_kernels(ok, "forward") == 7 and g.num_kernels(ok, "backward") == 12
    rws, saved, fws, bws = g.workspace_size(ok)
    M = 64 * 2
    # G13 kept in fp32, plus the transposed weight codes the backward reuses
    assert saved >= M * 2 * 128 * 4 + 8 * 3 * 128 * 128 * 33 // 32
    assert fws >= 64 * 128 + 8 * 3 * 128 * 128 + M * 128   # MXFP8 copies of x, W13, W2, A (A never stored unquantised)
    sz = ctypes.c_size_t(0)
    bad = g.Dims.of(64, 128, 64, 8, 2, "mxfp8")            # I must be a multiple of 128
    assert lib.moe_workspace_size(ctypes.byref(bad), ctypes.byref(sz), None, None, None) == 3


def test_router_projection_argument_errors():
    """moe_route_project / moe_router_backward validate on the host before any
    launch: fp32 mode unsupported, null and misaligned pointers, workspace."""
    g, lib = _lib()
    d = g.Dims.of(64, 128, 64, 8, 2, "bf16")
    r = _fake_routing(g)
    t = lambda i: _FakeTensor(0x7C0000000000 + i * 0x1000000)
    with pytest.raises(g.MoeError) as ei:
        g.route_project(g.Dims.of(64, 128, 64, 8, 2, "fp32"), t(0), t(1), t(2), r, t(3), stream=_NullStream())
    assert ei.value.status == 3
    with pytest.raises(g.MoeError) as ei:
        g.route_project(d, t(0), None, t(2), r, t(3), stream=_NullStream())
    assert ei.value.status == 1
    with pytest.raises(g.MoeError) as ei:
        g.route_project(d, t(0), _FakeTensor(0x7C0000000010), t(2), r, t(3), stream=_NullStream())
    assert ei.value.status == 4
    with pytest.raises(g.MoeError) as ei:
        g.route_project(d, t(0), t(1), t(2), r, _FakeTensor(0x7B0000000000, 1), stream=_NullStream())
    assert ei.value.status == 5
    with pytest.raises(g.MoeError) as ei:
        g.router_backward(d, r, t(0), t(1), t(2), None, t(4), stream=_NullStream())
    assert ei.value.status == 1
    with pytest.raises(g.MoeError) as ei:
        g.router_backward(g.Dims.of(64, 128, 64, 8, 2, "fp32"), r, t(0), t(1), t(2), t(3), t(4),
                          stream=_NullStream())
    assert ei.value.status == 3


def test_launch_status_is_the_launch_own():
    """A call that passes validation reaches its first launch; the status it
    returns is that launch's own.  On a machine without a GPU the launch fails
    and the call reports MOE_ERR_LAUNCH, while invalid arguments still return
    their validation status first (nothing is launched)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("checks the launch failure of a machine without a GPU")
    g, lib = _lib()
    d = g.Dims.of(64, 128, 64, 8, 2, "bf16")
    r = _fake_routing(g)
    c = r.c()
    logits, ws = 0x7E0000000000, 0x7D0000000000
    assert lib.moe_route(ctypes.byref(d), ctypes.c_void_p(logits), ctypes.byref(c), ctypes.c_void_p(ws), 16,
                         None) == 5
    assert lib.moe_route(ctypes.byref(d), ctypes.c_void_p(logits), ctypes.byref(c), ctypes.c_void_p(ws), 1 << 20,
                         None) == 6


def test_route_noalloc_limit_checked_before_launch():
    """moe_route_noalloc validates like moe_route and rejects shapes whose
    routing scratch exceeds the library's static array before any launch."""
    g, lib = _lib()
    r = _fake_routing(g)
    c = r.c()
    logits = ctypes.c_void_p(0x7E0000000000)
    big = g.Dims.of(131072, 64, 64, 512, 32, "bf16")          # 4 MiB of block partials
    assert g.workspace_size(big)[0] > 2 << 20
    assert lib.moe_route_noalloc(ctypes.byref(big), logits, ctypes.byref(c), None) == 5
    ok = g.Dims.of(64, 128, 64, 8, 2, "bf16")
    assert lib.moe_route_noalloc(ctypes.byref(ok), None, ctypes.byref(c), None) == 1
    assert lib.moe_route_noalloc(ctypes.byref(ok), ctypes.c_void_p(0x7E0000000004), ctypes.byref(c), None) == 4
    assert lib.moe_route_noalloc(ctypes.byref(g.Dims.of(64, 128, 64, 8, 9, "bf16")), logits, ctypes.byref(c),
                                 None) == 2


def test_weight_codes_sizes_and_errors():
    """moe_weight_codes_size: two transposed copies in fp8_bwd, four copies in
    mxfp8, unsupported without MXFP8 GEMMs; the cached calls validate before
    any launch."""
    g, lib = _lib()
    T, H, I, E, k = 64, 256, 128, 8, 2
    al = lambda n: (n + 255) // 256 * 256
    one = al(E * 2 * I * H) + al(E * 2 * I * H // 32) + al(E * H * I) + al(E * H * I // 32)
    assert g.weight_codes_size(g.Dims.of(T, H, I, E, k, "fp8_bwd")) == one
    assert g.weight_codes_size(g.Dims.of(T, H, I, E, k, "mxfp8")) == 2 * one
    sz = ctypes.c_size_t(0)
    assert lib.moe_weight_codes_size(ctypes.byref(g.Dims.of(T, H, I, E, k, "bf16")), ctypes.byref(sz)) == 3
    assert lib.moe_weight_codes_size(ctypes.byref(g.Dims.of(T, H, I, E, k, "mxfp8")), None) == 1
    t = lambda i: ctypes.c_void_p(0x7C0000000000 + i * 0x1000000)
    d8 = g.Dims.of(T, H, I, E, k, "fp8_bwd")
    q = lib.moe_quantize_weights
    assert q(ctypes.byref(g.Dims.of(T, H, I, E, k, "bf16")), t(0), t(1), t(2), 1 << 30, None) == 3
    assert q(ctypes.byref(d8), None, t(1), t(2), 1 << 30, None) == 1
    assert q(ctypes.byref(d8), t(0), t(1), ctypes.c_void_p(0x7C0000000010), 1 << 30, None) == 4
    assert q(ctypes.byref(d8), t(0), t(1), t(2), one - 1, None) == 5
    r = _fake_routing(g)
    c = r.c()
    fc, bc = lib.moe_forward_cached, lib.moe_backward_cached
    # forward_cached(dims, x, w13, w2, codes, routing, y, saved, ws, ws_bytes, stream)
    assert fc(ctypes.byref(g.Dims.of(T, H, I, E, k, "bf16")), t(0), t(1), t(2), t(3), ctypes.byref(c), t(4), t(5),
              t(6), 1 << 30, None) == 3
    assert fc(ctypes.byref(d8), t(0), t(1), t(2), None, ctypes.byref(c), t(4), t(5), t(6), 1 << 30, None) == 1
    assert fc(ctypes.byref(d8), t(0), t(1), t(2), ctypes.c_void_p(0x7C0000000010), ctypes.byref(c), t(4), t(5),
              t(6), 1 << 30, None) == 4
    assert fc(ctypes.byref(d8), t(0), t(1), t(2), t(3), ctypes.byref(c), t(4), t(5), t(6), 16, None) == 5
    # backward_cached(dims, dy, x, codes, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes, stream)
    assert bc(ctypes.byref(d8), t(0), t(1), None, ctypes.byref(c), t(4), t(5), t(6), t(7), t(8), None, t(9),
              1 << 30, None) == 1
    assert bc(ctypes.byref(d8), t(0), t(1), t(3), ctypes.byref(c), t(4), t(5), t(6), t(7), t(8), None, t(9),
              16, None) == 5
    assert bc(ctypes.byref(g.Dims.of(T, H, I, E, k, "bf16")), t(0), t(1), t(3), ctypes.byref(c), t(4), t(5), t(6),
              t(7), t(8), None, t(9), 1 << 30, None) == 3

def test_wgrad_chunk_rows():
    """The weight-gradient chunk size is a positive multiple of the 128-row
    MXFP8 K tile (chunk boundaries must fall on K tiles)."""
    import grouped_gemm_layer_amd as g
    kc = g.wgrad_chunk_rows()
    assert kc > 0 and kc % 128 == 0
