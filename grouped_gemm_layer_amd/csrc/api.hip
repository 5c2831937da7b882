// C ABI of the MoE expert layer: argument validation, workspace carving and
// the launch sequence of each call.  The only host work of every call; no
// allocation, no host synchronisation, no device-to-host copy.
#include "../../include/moe.h"
#include "moe_internal.h"

#include <stdint.h>

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

struct Sizes {
  size_t route_ws, saved, fwd_ws, bwd_ws;
  // carving offsets
  size_t r_partials, r_bases;
  size_t f_tile_e, f_tile_r, f_tile_x, f_A, f_O;
  size_t f_qx, f_sx, f_qw13, f_sw13, f_qa, f_sa, f_qw2, f_sw2;   // mxfp8 forward operands
  size_t b_tile_e, b_tile_r, b_tile_x, b_wg_order, b_wg_cstart, b_wg_slot0, b_wg_xq, b_wpart13, b_wpart2;
  size_t b_dG13, b_Ag, b_dXp, b_part;
  // fp8_bwd: MXFP8 operand copies of the backward GEMMs (codes, scales)
  size_t Mp;
  // mxfp8: the transposed weight operands of the backward, kept in `saved` by the forward
  size_t sv_qw13t, sv_sw13t, sv_qw2t, sv_sw2t;
  size_t q_pad, q_dy, s_dy, q_w2t, s_w2t, q_dg, s_dg, q_w13t, s_w13t;
  size_t q_dyt, s_dyt, q_agt, s_agt, q_dgt, s_dgt, q_xt, s_xt;
};

moe_status check_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->T <= 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->k <= 0 || d->k > d->E) return MOE_ERR_DIMS;
  if ((int64_t)d->T * d->k > INT32_MAX) return MOE_ERR_DIMS;
  if ((int64_t)d->E * 2 * d->I * d->H > ((int64_t)1 << 40)) return MOE_ERR_DIMS;
  if (d->mode != MOE_MODE_FP32 && d->mode != MOE_MODE_BF16 && d->mode != MOE_MODE_MXFP8 &&
      d->mode != MOE_MODE_FP8_BWD)
    return MOE_ERR_UNSUPPORTED;
  if (d->H % 64 != 0 || d->I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (mx8_backward(d->mode) && d->H % MX_KTILE != 0) return MOE_ERR_UNSUPPORTED;
  if (mx8_forward(d->mode) && d->I % MX_KTILE != 0) return MOE_ERR_UNSUPPORTED;
  if (d->E > 512 || d->k > 32) return MOE_ERR_UNSUPPORTED;
  // every per-operand buffer is addressed with 32-bit byte offsets
  const int64_t M = (int64_t)d->T * d->k;
  const int64_t wide = d->H > 2 * d->I ? d->H : 2 * d->I;
  const int64_t es = d->mode == MOE_MODE_FP32 ? 4 : 2;
  if (M * wide * es >= ((int64_t)1 << 31) || (int64_t)2 * d->I * d->H * es >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  if (mx8_backward(d->mode) && (int64_t)mx_token_capacity((size_t)M, d->E) * wide >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Sizes compute_sizes(const moe_dims* d) {
  Sizes s{};
  const size_t M = (size_t)d->T * d->k;
  const size_t es = (d->mode == MOE_MODE_FP32) ? 4 : 2;
  const size_t max_tiles = (size_t)max_row_tiles((int)M, d->E, fwd_row_tile_m(d->mode));
  const size_t max_tiles_b = (size_t)max_row_tiles((int)M, d->E, bwd_row_tile_m(d->mode, d->H, d->I));
  const size_t nblk = (size_t)route_num_blocks((int)M);
  size_t o = 0;
  s.r_partials = o; o += align_up(nblk * d->E * 4);
  s.r_bases = o;    o += align_up(nblk * d->E * 4);
  s.route_ws = o;
  // the MXFP8 backward keeps G13 in fp32: its derivatives are quantised unrounded
  s.saved = align_up(M * 2 * d->I * (mx8_backward(d->mode) ? 4 : es));
  if (mx8_forward(d->mode)) {   // weights are quantised both ways once, in the forward
    const size_t w13 = (size_t)d->E * 2 * d->I * d->H, w2 = (size_t)d->E * d->H * d->I;
    s.sv_qw13t = s.saved; s.saved += align_up(w13);
    s.sv_sw13t = s.saved; s.saved += align_up(w13 / 32);
    s.sv_qw2t = s.saved;  s.saved += align_up(w2);
    s.sv_sw2t = s.saved;  s.saved += align_up(w2 / 32);
  }
  o = 0;
  s.f_tile_e = o; o += align_up(max_tiles * 4);
  s.f_tile_r = o; o += align_up(max_tiles * 4);
  s.f_tile_x = o; o += align_up(((size_t)d->E + 1) * 4);
  if (!mx8_forward(d->mode)) {   // the mxfp8 forward quantises A in the epilogue instead
    s.f_A = o; o += align_up(M * d->I * es);
  }
  s.f_O = o;      o += align_up(M * d->H * es);
  if (mx8_forward(d->mode)) {
    const size_t T = d->T, H = d->H, I = d->I, E = d->E;
    auto take = [&](size_t& at_, size_t bytes) { at_ = o; o += align_up(bytes); };
    take(s.f_qx, T * H);          take(s.f_sx, T * H / 32);
    take(s.f_qw13, E * 2 * I * H); take(s.f_sw13, E * 2 * I * H / 32);
    take(s.f_qa, M * I);          take(s.f_sa, M * I / 32);
    take(s.f_qw2, E * H * I);     take(s.f_sw2, E * H * I / 32);
  }
  s.fwd_ws = o;
  o = 0;
  s.b_tile_e = o; o += align_up(max_tiles_b * 4);
  s.b_tile_r = o; o += align_up(max_tiles_b * 4);
  s.b_tile_x = o; o += align_up(((size_t)d->E + 1) * 4);
  s.b_wg_order = o;  o += align_up((size_t)d->E * 4);
  s.b_wg_cstart = o; o += align_up(((size_t)d->E + 1) * 4);
  s.b_wg_slot0 = o;  o += align_up((size_t)d->E * 4);
  s.b_wg_xq = o;     o += align_up((size_t)wgrad_queue_slots(wgrad_max_chunks((int)M, d->E)) * 4);
  if (d->mode != MOE_MODE_FP32) {   // fp32 partial results of the chunks c > 0 of split experts
    const size_t slots = wgrad_max_slots(M);
    s.b_wpart13 = o; o += align_up(slots * 2 * d->I * d->H * 4);
    s.b_wpart2 = o;  o += align_up(slots * d->H * d->I * 4);
  }
  if (!mx8_backward(d->mode)) {   // the MXFP8 backward quantises them in the dgrad epilogue instead
    s.b_dG13 = o; o += align_up(M * 2 * d->I * es);
    s.b_Ag = o;   o += align_up(M * d->I * es);
  }
  s.b_dXp = o;    o += align_up(M * d->H * es);
  s.b_part = o;   o += align_up((size_t)dgrad2_parts(d->mode, d->I) * M * 4);
  if (mx8_backward(d->mode)) {
    const size_t T = d->T, H = d->H, I = d->I, E = d->E;
    const size_t Mp = mx_token_capacity(M, d->E);
    s.Mp = Mp;
    auto take = [&](size_t& at_, size_t bytes) { at_ = o; o += align_up(bytes); };
    take(s.q_pad, (E + 1) * 4);
    take(s.q_dy, T * H);          take(s.s_dy, T * H / 32);
    if (!mx8_forward(d->mode)) {   // else in `saved`
      take(s.q_w2t, E * I * H);     take(s.s_w2t, E * I * H / 32);
      take(s.q_w13t, E * H * 2 * I); take(s.s_w13t, E * H * 2 * I / 32);
    }
    take(s.q_dg, M * 2 * I);      take(s.s_dg, M * 2 * I / 32);
    take(s.q_dyt, H * Mp);        take(s.s_dyt, H * Mp / 32);
    take(s.q_agt, I * Mp);        take(s.s_agt, I * Mp / 32);
    take(s.q_dgt, 2 * I * Mp);    take(s.s_dgt, 2 * I * Mp / 32);
    take(s.q_xt, H * Mp);         take(s.s_xt, H * Mp / 32);
  }
  s.bwd_ws = o;
  return s;
}

// Layout of the caller's cache of MXFP8 weight copies (moe_quantize_weights):
// the forward's row-wise copies (MOE_MODE_MXFP8) and the backward's transposed
// copies (both fp8 modes), codes then scales, each 256-byte aligned.
struct WCodes {
  size_t qw13, sw13, qw2, sw2, qw13t, sw13t, qw2t, sw2t, bytes;
};
WCodes wcodes_layout(const moe_dims* d) {
  WCodes w{};
  const size_t n13 = (size_t)d->E * 2 * d->I * d->H, n2 = (size_t)d->E * d->H * d->I;
  size_t o = 0;
  if (mx8_forward(d->mode)) {
    w.qw13 = o; o += align_up(n13);
    w.sw13 = o; o += align_up(n13 / 32);
    w.qw2 = o;  o += align_up(n2);
    w.sw2 = o;  o += align_up(n2 / 32);
  }
  if (mx8_backward(d->mode)) {
    w.qw13t = o; o += align_up(n13);
    w.sw13t = o; o += align_up(n13 / 32);
    w.qw2t = o;  o += align_up(n2);
    w.sw2t = o;  o += align_up(n2 / 32);
  }
  w.bytes = o;
  return w;
}

moe_status check_routing(const moe_routing* r) {
  if (!r) return MOE_ERR_NULL;
  if (!r->topk_idx || !r->gate || !r->counts || !r->offsets || !r->sorted_to_flat || !r->flat_to_sorted)
    return MOE_ERR_NULL;
  if (!aligned(r->topk_idx) || !aligned(r->gate) || !aligned(r->counts) || !aligned(r->offsets) ||
      !aligned(r->sorted_to_flat) || !aligned(r->flat_to_sorted))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

LayerArgs base_args(const moe_dims* d, const moe_routing* r) {
  LayerArgs a{};
  a.T = d->T; a.H = d->H; a.I = d->I; a.E = d->E; a.k = d->k; a.M = d->T * d->k;
  a.offsets = r->offsets;
  a.s2f = r->sorted_to_flat;
  a.f2s = r->flat_to_sorted;
  a.gate = r->gate;
  return a;
}

inline hipError_t gemm(bool bf16, GemmKind kind, const LayerArgs& a, hipStream_t s) {
  return bf16 ? launch_gemm_bf16(kind, a, s) : launch_gemm_fp32(kind, a, s);
}

Mx8Args mx8_args(const moe_dims* d, const Sizes& s, void* ws, const void* saved) {
  auto u8 = [&](size_t off) { return reinterpret_cast<const uint8_t*>(at(ws, off)); };
  auto sv = [&](size_t off) { return static_cast<const uint8_t*>(saved) + off; };
  Mx8Args q{};
  q.pad_off = reinterpret_cast<const int32_t*>(at(ws, s.q_pad));
  q.Mp = (int)s.Mp;
  q.qdy = u8(s.q_dy);     q.sdy = u8(s.s_dy);
  q.qdg = u8(s.q_dg);     q.sdg = u8(s.s_dg);
  if (mx8_forward(d->mode)) {
    q.qw2t = sv(s.sv_qw2t);   q.sw2t = sv(s.sv_sw2t);
    q.qw13t = sv(s.sv_qw13t); q.sw13t = sv(s.sv_sw13t);
  } else {
    q.qw2t = u8(s.q_w2t);   q.sw2t = u8(s.s_w2t);
    q.qw13t = u8(s.q_w13t); q.sw13t = u8(s.s_w13t);
  }
  q.qdyt = u8(s.q_dyt);   q.sdyt = u8(s.s_dyt);
  q.qagt = u8(s.q_agt);   q.sagt = u8(s.s_agt);
  q.qdgt = u8(s.q_dgt);   q.sdgt = u8(s.s_dgt);
  q.qxt = u8(s.q_xt);     q.sxt = u8(s.s_xt);
  return q;
}
inline uint8_t* mut(const uint8_t* p) { return const_cast<uint8_t*>(p); }

// Optional event marks for benchmarking: events[0] before the first kernel,
// events[i + 1] after kernel i (stream-ordered; no synchronisation).
struct Marks {
  hipEvent_t* ev;
  int n;
  int i;
  hipStream_t s;
  hipError_t mark() {
    if (ev && i < n) return hipEventRecord(ev[i++], s);
    return hipSuccess;
  }
};

// kernels per call, in launch order
constexpr int kRouteKernels = 4;      // topk+gate, histogram, scan, scatter
constexpr int kForwardKernels = 4;    // tile table, GEMM1+SwiGLU, GEMM2, combine
// mxfp8: tile table, quant x, quant W13, GEMM1+SwiGLU+quant A, quant W2, GEMM2, combine
constexpr int kForwardKernelsMx8 = 7;
inline int forward_kernels(int mode) { return mx8_forward(mode) ? kForwardKernelsMx8 : kForwardKernels; }
// tile table, dgrad W2 + dSwiGLU, dgrad W13, unpermute, router, wgrad W2, wgrad W13,
// and (bf16) the ordered split-K completion of the weight gradients
constexpr int kBackwardKernels = 7;
// MXFP8 backward: tile table, padded offsets, quant W2^T, quant dY, dgrad W2 +
// dSwiGLU + quant dG13 (row and token blocks) and gate*A (token blocks),
// quant W13^T, dgrad W13, unpermute, router, quant dY^T, wgrad W2, quant x^T,
// wgrad W13, split-K completion
constexpr int kBackwardKernelsMx8 = 14;
// MOE_MODE_MXFP8: the same without the two weight quantisers (the forward saved W2^T and W13^T codes)
inline int backward_kernels(int mode) {
  return mx8_forward(mode) ? kBackwardKernelsMx8 - 2
         : mx8_backward(mode) ? kBackwardKernelsMx8
         : mode == MOE_MODE_FP32 ? kBackwardKernels : kBackwardKernels + 1;
}

// wcodes: the caller's MXFP8 weight copies (moe_quantize_weights), or null
// when the call quantises the weights itself
moe_status forward_impl(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                        const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                        hipStream_t stream, Marks mk, bool recompute = false, const void* wcodes = nullptr);
moe_status backward_impl(const moe_dims* dims, const void* dy, const void* x, const void* w13, const void* w2,
                         const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                         float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream, Marks mk,
                         bool accumulate = false, const void* wcodes = nullptr);

}  // namespace

extern "C" {

moe_status moe_workspace_size(const moe_dims* dims, size_t* route_ws, size_t* saved, size_t* fwd_ws,
                              size_t* bwd_ws) {
  const moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  const Sizes s = compute_sizes(dims);
  if (route_ws) *route_ws = s.route_ws;
  if (saved) *saved = s.saved;
  if (fwd_ws) *fwd_ws = s.fwd_ws;
  if (bwd_ws) *bwd_ws = s.bwd_ws;
  return MOE_OK;
}

moe_status moe_route(const moe_dims* dims, const float* logits, const moe_routing* out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_routing(out)) != MOE_OK) return st;
  if (!logits || !ws) return MOE_ERR_NULL;
  if (!aligned(logits) || !aligned(ws)) return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  if (ws_bytes < s.route_ws) return MOE_ERR_WORKSPACE;
  const hipError_t e = launch_route(logits, dims->T, dims->E, dims->k, out->topk_idx, out->gate, out->counts,
                                    out->offsets, out->sorted_to_flat, out->flat_to_sorted,
                                    reinterpret_cast<int32_t*>(at(ws, s.r_partials)),
                                    reinterpret_cast<int32_t*>(at(ws, s.r_bases)), stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status moe_route_noalloc(const moe_dims* dims, const float* logits, const moe_routing* out,
                             hipStream_t stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_routing(out)) != MOE_OK) return st;
  if (!logits) return MOE_ERR_NULL;
  if (!aligned(logits)) return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  static_assert(MOE_ROUTE_NOALLOC_MAX_BYTES == ROUTE_SCRATCH_BYTES, "header and library agree on the scratch size");
  if (s.route_ws > ROUTE_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;   // this device's address of the library's routing scratch
  if (route_scratch_ptr(&ws) != hipSuccess) return MOE_ERR_LAUNCH;
  const hipError_t e = launch_route(logits, dims->T, dims->E, dims->k, out->topk_idx, out->gate, out->counts,
                                    out->offsets, out->sorted_to_flat, out->flat_to_sorted,
                                    reinterpret_cast<int32_t*>(at(ws, s.r_partials)),
                                    reinterpret_cast<int32_t*>(at(ws, s.r_bases)), stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status moe_route_project(const moe_dims* dims, const void* x, const void* w_router, float* logits,
                             const moe_routing* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->mode == MOE_MODE_FP32) return MOE_ERR_UNSUPPORTED;
  if ((st = check_routing(out)) != MOE_OK) return st;
  if (!x || !w_router || !logits || !ws) return MOE_ERR_NULL;
  if (!aligned(x) || !aligned(w_router) || !aligned(logits) || !aligned(ws)) return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  if (ws_bytes < s.route_ws) return MOE_ERR_WORKSPACE;
  hipError_t e = launch_router_logits(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router), dims->T,
                                      dims->H, dims->E, logits, stream);
  if (e == hipSuccess)
    e = launch_route(logits, dims->T, dims->E, dims->k, out->topk_idx, out->gate, out->counts, out->offsets,
                     out->sorted_to_flat, out->flat_to_sorted, reinterpret_cast<int32_t*>(at(ws, s.r_partials)),
                     reinterpret_cast<int32_t*>(at(ws, s.r_bases)), stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status moe_router_backward(const moe_dims* dims, const moe_routing* routing, const float* dlogits,
                               const void* x, const void* w_router, void* dx, float* dw_router,
                               hipStream_t stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->mode == MOE_MODE_FP32) return MOE_ERR_UNSUPPORTED;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  if (!dlogits || !x || !w_router || !dx || !dw_router) return MOE_ERR_NULL;
  if (!aligned(dlogits) || !aligned(x) || !aligned(w_router) || !aligned(dx) || !aligned(dw_router))
    return MOE_ERR_ALIGN;
  const hipError_t e = launch_router_project_bwd(
      dlogits, routing->topk_idx, routing->offsets, routing->sorted_to_flat, static_cast<const bf16_t*>(x),
      static_cast<const bf16_t*>(w_router), dims->T, dims->H, dims->E, dims->k, static_cast<bf16_t*>(dx), dw_router,
      stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// recompute: the second forward of activation checkpointing, which restores
// `saved` for the backward and skips what only produces y (GEMM W2, combine)
moe_status forward_impl(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                        const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                        hipStream_t stream, Marks mk, bool recompute, const void* wcodes) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  // saved may be NULL (not in the recompute): the forward then keeps nothing for a backward
  if (!x || !w13 || !w2 || (!y && !recompute) || (!saved && recompute) || !ws) return MOE_ERR_NULL;
  if (!aligned(x) || !aligned(w13) || !aligned(w2) || !aligned(y) || !aligned(saved) || !aligned(ws))
    return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  if (ws_bytes < s.fwd_ws) return MOE_ERR_WORKSPACE;
  const bool bf16 = dims->mode != MOE_MODE_FP32;
  LayerArgs a = base_args(dims, routing);
  a.x = x; a.w13 = w13; a.w2 = w2;
  a.G13 = saved;
  a.g13_f32 = mx8_backward(dims->mode);
  a.A = (mx8_forward(dims->mode) || recompute) ? nullptr : at(ws, s.f_A);
  a.O = at(ws, s.f_O);
  int32_t* te = reinterpret_cast<int32_t*>(at(ws, s.f_tile_e));
  int32_t* tr = reinterpret_cast<int32_t*>(at(ws, s.f_tile_r));
  int32_t* tx = reinterpret_cast<int32_t*>(at(ws, s.f_tile_x));
  a.tile_expert = te; a.tile_row0 = tr; a.expert_tile0 = tx;
  const int bm = fwd_row_tile_m(dims->mode);
  hipError_t e = mk.mark();
  auto step = [&](hipError_t r) {   // record kernel completion, keep the first error
    if (e == hipSuccess) e = r;
    if (e == hipSuccess) e = mk.mark();
  };
  step(launch_tile_table(routing->offsets, dims->E, bm, max_row_tiles(a.M, a.E, bm), te, tr, tx, WgradList{},
                         stream));
  if (mx8_forward(dims->mode)) {
    auto u8 = [&](size_t off) { return reinterpret_cast<uint8_t*>(at(ws, off)); };
    Mx8Args q{};
    q.qx = u8(s.f_qx);     q.sx = u8(s.f_sx);
    q.qw13 = u8(s.f_qw13); q.sw13 = u8(s.f_sw13);
    q.qa = u8(s.f_qa);     q.sa = u8(s.f_sa);
    if (!recompute) { a.q_a = u8(s.f_qa); a.q_sa = u8(s.f_sa); }
    q.qw2 = u8(s.f_qw2);   q.sw2 = u8(s.f_sw2);
    if (wcodes) {   // the caller's copies: no weight quantisation in this call
      const WCodes wc = wcodes_layout(dims);
      auto cp = [&](size_t off) { return static_cast<const uint8_t*>(wcodes) + off; };
      q.qw13 = cp(wc.qw13); q.sw13 = cp(wc.sw13);
      q.qw2 = cp(wc.qw2);   q.sw2 = cp(wc.sw2);
    }
    const bf16_t* x16 = static_cast<const bf16_t*>(x);
    if (e == hipSuccess) step(launch_mx_quant_rows(x16, a.T, a.H, nullptr, 1, u8(s.f_qx), u8(s.f_sx), stream));
    auto svp = [&](size_t off) { return static_cast<uint8_t*>(saved) + off; };
    // each weight quantised both ways (the transposed copy, for the backward,
    // into `saved`), or only along its rows when nothing is kept
    auto quant_w = [&](const void* w, int rows_per_e, int cols, size_t sv_q, size_t sv_s, size_t f_q, size_t f_s) {
      const bf16_t* w16 = static_cast<const bf16_t*>(w);
      if (saved)
        step(launch_mx_quant_both(w16, a.E, rows_per_e, cols, svp(sv_q), svp(sv_s), u8(f_q), u8(f_s), stream));
      else
        step(launch_mx_quant_rows(w16, a.E * rows_per_e, cols, nullptr, 1, u8(f_q), u8(f_s), stream));
    };
    if (e == hipSuccess && !wcodes) quant_w(w13, 2 * a.I, a.H, s.sv_qw13t, s.sv_sw13t, s.f_qw13, s.f_sw13);
    if (e == hipSuccess) step(launch_gemm_mx8(KIND_FWD1, a, q, stream));
    // the transposed W2 copy in `saved` is the backward's, so the recompute keeps it
    if (e == hipSuccess && !wcodes) quant_w(w2, a.H, a.I, s.sv_qw2t, s.sv_sw2t, s.f_qw2, s.f_sw2);
    if (e == hipSuccess && !recompute) step(launch_gemm_mx8(KIND_FWD2, a, q, stream));
  } else {
    if (e == hipSuccess) step(gemm(bf16, KIND_FWD1, a, stream));
    if (e == hipSuccess && !recompute) step(gemm(bf16, KIND_FWD2, a, stream));
  }
  if (e == hipSuccess && !recompute) {
    if (bf16)
      e = launch_combine<bf16_t>(static_cast<const bf16_t*>(a.O), a.f2s, a.gate, a.T, a.k, a.H,
                                 static_cast<bf16_t*>(y), stream);
    else
      e = launch_combine<float>(static_cast<const float*>(a.O), a.f2s, a.gate, a.T, a.k, a.H,
                                static_cast<float*>(y), stream);
    if (e == hipSuccess) e = mk.mark();
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status backward_impl(const moe_dims* dims, const void* dy, const void* x, const void* w13, const void* w2,
                         const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                         float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream, Marks mk,
                         bool accumulate, const void* wcodes) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  // with the caller's weight copies the bf16 weights are not read
  if (!dy || !x || (!wcodes && (!w13 || !w2)) || !saved || !dx || !dw13 || !dw2 || !dgate || !ws)
    return MOE_ERR_NULL;
  if (!aligned(dy) || !aligned(x) || !aligned(w13) || !aligned(w2) || !aligned(saved) || !aligned(dx) ||
      !aligned(dw13) || !aligned(dw2) || !aligned(dgate) || !aligned(ws) || (dlogits && !aligned(dlogits)))
    return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  if (ws_bytes < s.bwd_ws) return MOE_ERR_WORKSPACE;
  const bool bf16 = dims->mode != MOE_MODE_FP32;
  LayerArgs a = base_args(dims, routing);
  a.x = x; a.w13 = w13; a.w2 = w2; a.dy = dy;
  a.G13 = const_cast<void*>(saved);
  const bool mx8 = mx8_backward(dims->mode);
  a.dG13 = mx8 ? nullptr : at(ws, s.b_dG13);
  a.Ag = mx8 ? nullptr : at(ws, s.b_Ag);
  a.dXp = at(ws, s.b_dXp);
  a.dgate_part = reinterpret_cast<float*>(at(ws, s.b_part));
  a.dw13 = dw13;
  a.dw2 = dw2;
  a.wgrad_acc = accumulate ? 1 : 0;
  int32_t* te = reinterpret_cast<int32_t*>(at(ws, s.b_tile_e));
  int32_t* tr = reinterpret_cast<int32_t*>(at(ws, s.b_tile_r));
  int32_t* tx = reinterpret_cast<int32_t*>(at(ws, s.b_tile_x));
  a.tile_expert = te; a.tile_row0 = tr; a.expert_tile0 = tx;
  // weight-gradient work list (bf16 and MXFP8 kernels; the fp32 kernels take whole experts)
  const bool split = bf16;
  WgradList wg{};
  if (split) {
    wg.order = reinterpret_cast<int32_t*>(at(ws, s.b_wg_order));
    wg.cstart = reinterpret_cast<int32_t*>(at(ws, s.b_wg_cstart));
    wg.slot0 = reinterpret_cast<int32_t*>(at(ws, s.b_wg_slot0));
    wg.xq = reinterpret_cast<int32_t*>(at(ws, s.b_wg_xq));
    a.wg_order = wg.order; a.wg_cstart = wg.cstart; a.wg_slot0 = wg.slot0; a.wg_xq = wg.xq;
    a.wpart13 = reinterpret_cast<float*>(at(ws, s.b_wpart13));
    a.wpart2 = reinterpret_cast<float*>(at(ws, s.b_wpart2));
  }
  const int bm = bwd_row_tile_m(dims->mode, dims->H, dims->I);
  Mx8Args q = mx8 ? mx8_args(dims, s, ws, saved) : Mx8Args{};
  if (mx8 && wcodes) {   // the caller's transposed weight copies
    const WCodes wc = wcodes_layout(dims);
    auto cp = [&](size_t off) { return static_cast<const uint8_t*>(wcodes) + off; };
    q.qw2t = cp(wc.qw2t);   q.sw2t = cp(wc.sw2t);
    q.qw13t = cp(wc.qw13t); q.sw13t = cp(wc.sw13t);
  }
  const bf16_t* dy16 = static_cast<const bf16_t*>(dy);
  const bf16_t* x16 = static_cast<const bf16_t*>(x);
  // activation-gradient chain first; the weight gradients do not feed it
  hipError_t e = mk.mark();
  auto step = [&](hipError_t r) {   // record kernel completion, keep the first error
    if (e == hipSuccess) e = r;
    if (e == hipSuccess) e = mk.mark();
  };
  step(launch_tile_table(routing->offsets, dims->E, bm, max_row_tiles(a.M, a.E, bm), te, tr, tx, wg, stream));
  if (mx8) {
    // the dgrad epilogue of W2 places its token blocks at the padded offsets
    if (e == hipSuccess) step(launch_pad_offsets(a.offsets, a.E, const_cast<int32_t*>(q.pad_off), stream));
    // mxfp8: the forward saved W2^T and W13^T codes; cached: the caller's copies
    const bool wq = !mx8_forward(dims->mode) && !wcodes;
    if (e == hipSuccess && wq)
      step(launch_mx_quant_cols_t(static_cast<const bf16_t*>(w2), a.E, a.H, a.I, mut(q.qw2t), mut(q.sw2t), stream));
    if (e == hipSuccess) step(launch_mx_quant_rows(dy16, a.T, a.H, nullptr, 1, mut(q.qdy), mut(q.sdy), stream));
    if (e == hipSuccess) step(launch_gemm_mx8(KIND_DGRAD2, a, q, stream));
    if (e == hipSuccess && wq)
      step(launch_mx_quant_cols_t(static_cast<const bf16_t*>(w13), a.E, 2 * a.I, a.H, mut(q.qw13t), mut(q.sw13t),
                                  stream));
    if (e == hipSuccess) step(launch_gemm_mx8(KIND_DGRAD1, a, q, stream));
  } else {
    if (e == hipSuccess) step(gemm(bf16, KIND_DGRAD2, a, stream));
    if (e == hipSuccess) step(gemm(bf16, KIND_DGRAD1, a, stream));
  }
  if (e == hipSuccess) {
    if (bf16)
      step(launch_combine<bf16_t>(static_cast<const bf16_t*>(a.dXp), a.f2s, nullptr, a.T, a.k, a.H,
                                  static_cast<bf16_t*>(dx), stream));
    else
      step(launch_combine<float>(static_cast<const float*>(a.dXp), a.f2s, nullptr, a.T, a.k, a.H,
                                 static_cast<float*>(dx), stream));
  }
  if (e == hipSuccess)
    step(launch_router_bwd(a.dgate_part, dgrad2_parts(dims->mode, a.I), a.f2s, a.gate, routing->topk_idx, a.T,
                           a.k, a.E, a.M, dgate, dlogits, stream));
  if (mx8) {
    const int32_t* pad = q.pad_off;
    if (e == hipSuccess)
      step(launch_mx_quant_tokens_t(dy16, a.H, a.s2f, a.k, a.offsets, pad, a.E, q.Mp, mut(q.qdyt), mut(q.sdyt),
                                    stream));
    if (e == hipSuccess) step(launch_gemm_mx8(KIND_WGRAD2, a, q, stream));
    if (e == hipSuccess)
      step(launch_mx_quant_tokens_t(x16, a.H, a.s2f, a.k, a.offsets, pad, a.E, q.Mp, mut(q.qxt), mut(q.sxt),
                                    stream));
    if (e == hipSuccess) step(launch_gemm_mx8(KIND_WGRAD1, a, q, stream));
  } else {
    if (e == hipSuccess) step(gemm(bf16, KIND_WGRAD2, a, stream));
    if (e == hipSuccess) step(gemm(bf16, KIND_WGRAD1, a, stream));
  }
  if (split && e == hipSuccess) step(launch_wgrad_reduce(a, stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                       const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return forward_impl(dims, x, w13, w2, routing, y, saved, ws, ws_bytes, stream, Marks{nullptr, 0, 0, stream});
}

moe_status moe_forward_recompute(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                                 const moe_routing* routing, void* saved, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  return forward_impl(dims, x, w13, w2, routing, nullptr, saved, ws, ws_bytes, stream,
                      Marks{nullptr, 0, 0, stream}, true);
}

moe_status moe_backward(const moe_dims* dims, const void* dy, const void* x, const void* w13, const void* w2,
                        const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                        float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream) {
  return backward_impl(dims, dy, x, w13, w2, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes, stream,
                       Marks{nullptr, 0, 0, stream});
}

int moe_num_kernels(const moe_dims* dims, int which) {
  if (check_dims(dims) != MOE_OK) return -1;
  return which == 0 ? kRouteKernels : which == 1 ? forward_kernels(dims->mode) : which == 2 ? backward_kernels(dims->mode) : -1;
}

moe_status moe_forward_timed(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                             const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                             hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!events) return MOE_ERR_NULL;
  if (check_dims(dims) == MOE_OK && n_events < forward_kernels(dims->mode) + 1) return MOE_ERR_DIMS;
  return forward_impl(dims, x, w13, w2, routing, y, saved, ws, ws_bytes, stream,
                      Marks{events, n_events, 0, stream});
}

moe_status moe_backward_accumulate(const moe_dims* dims, const void* dy, const void* x, const void* w13,
                                   const void* w2, const moe_routing* routing, const void* saved, void* dx,
                                   float* dw13, float* dw2, float* dgate, float* dlogits, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return backward_impl(dims, dy, x, w13, w2, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes, stream,
                       Marks{nullptr, 0, 0, stream}, true);
}

moe_status moe_backward_timed(const moe_dims* dims, const void* dy, const void* x, const void* w13,
                              const void* w2, const moe_routing* routing, const void* saved, void* dx,
                              float* dw13, float* dw2, float* dgate, float* dlogits, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!events) return MOE_ERR_NULL;
  if (check_dims(dims) == MOE_OK && n_events < backward_kernels(dims->mode) + 1) return MOE_ERR_DIMS;
  return backward_impl(dims, dy, x, w13, w2, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes, stream,
                       Marks{events, n_events, 0, stream});
}

moe_status moe_weight_codes_size(const moe_dims* dims, size_t* bytes) {
  const moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  if (!mx8_backward(dims->mode)) return MOE_ERR_UNSUPPORTED;
  *bytes = wcodes_layout(dims).bytes;
  return MOE_OK;
}

moe_status moe_quantize_weights(const moe_dims* dims, const void* w13, const void* w2, void* codes, size_t bytes,
                                hipStream_t stream) {
  const moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!mx8_backward(dims->mode)) return MOE_ERR_UNSUPPORTED;
  if (!w13 || !w2 || !codes) return MOE_ERR_NULL;
  if (!aligned(w13) || !aligned(w2) || !aligned(codes)) return MOE_ERR_ALIGN;
  const WCodes wc = wcodes_layout(dims);
  if (bytes < wc.bytes) return MOE_ERR_WORKSPACE;
  auto cp = [&](size_t off) { return static_cast<uint8_t*>(codes) + off; };
  const bf16_t* w13_16 = static_cast<const bf16_t*>(w13);
  const bf16_t* w2_16 = static_cast<const bf16_t*>(w2);
  const int E = dims->E, H = dims->H, I = dims->I;
  hipError_t e;
  if (mx8_forward(dims->mode)) {   // both copies of each weight from one read
    e = launch_mx_quant_both(w13_16, E, 2 * I, H, cp(wc.qw13t), cp(wc.sw13t), cp(wc.qw13), cp(wc.sw13), stream);
    if (e == hipSuccess)
      e = launch_mx_quant_both(w2_16, E, H, I, cp(wc.qw2t), cp(wc.sw2t), cp(wc.qw2), cp(wc.sw2), stream);
  } else {                         // fp8_bwd: the backward's transposed copies only
    e = launch_mx_quant_cols_t(w13_16, E, 2 * I, H, cp(wc.qw13t), cp(wc.sw13t), stream);
    if (e == hipSuccess) e = launch_mx_quant_cols_t(w2_16, E, H, I, cp(wc.qw2t), cp(wc.sw2t), stream);
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status moe_forward_cached(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                              const void* codes, const moe_routing* routing, void* y, void* saved, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!mx8_backward(dims->mode)) return MOE_ERR_UNSUPPORTED;
  if (!codes) return MOE_ERR_NULL;
  if (!aligned(codes)) return MOE_ERR_ALIGN;
  return forward_impl(dims, x, w13, w2, routing, y, saved, ws, ws_bytes, stream, Marks{nullptr, 0, 0, stream}, false,
                      codes);
}

moe_status moe_backward_cached(const moe_dims* dims, const void* dy, const void* x, const void* codes,
                               const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                               float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream) {
  const moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!mx8_backward(dims->mode)) return MOE_ERR_UNSUPPORTED;
  if (!codes) return MOE_ERR_NULL;
  if (!aligned(codes)) return MOE_ERR_ALIGN;
  return backward_impl(dims, dy, x, nullptr, nullptr, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes,
                       stream, Marks{nullptr, 0, 0, stream}, false, codes);
}

moe_status moe_mxfp8_quantize(const void* src, int32_t rows, int32_t cols, int32_t along, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  if (!src || !codes || !scales) return MOE_ERR_NULL;
  if (rows <= 0 || cols <= 0 || (along != 0 && along != 1)) return MOE_ERR_DIMS;
  if (along == 1 && cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (along == 0 && rows % MX_KTILE != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)rows * cols * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!aligned(src) || !aligned(codes) || !aligned(scales)) return MOE_ERR_ALIGN;
  const bf16_t* s16 = static_cast<const bf16_t*>(src);
  const hipError_t e = along == 1 ? launch_mx_quant_rows(s16, rows, cols, nullptr, 1, codes, scales, stream)
                                  : launch_mx_quant_cols_t(s16, 1, rows, cols, codes, scales, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status moe_mxfp8_quantize_grouped(const void* src, int32_t rows, int32_t cols, const int32_t* offsets,
                                      int32_t E, int32_t capacity, int32_t* pad_off, uint8_t* codes,
                                      uint8_t* scales, hipStream_t stream) {
  if (!src || !offsets || !pad_off || !codes || !scales) return MOE_ERR_NULL;
  if (rows <= 0 || cols <= 0 || E <= 0) return MOE_ERR_DIMS;
  if (E > 512 || capacity % MX_KTILE != 0 || (size_t)capacity < mx_token_capacity((size_t)rows, E))
    return MOE_ERR_UNSUPPORTED;
  if ((int64_t)rows * cols * 2 >= ((int64_t)1 << 31) || (int64_t)capacity * cols >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(src) || !aligned(offsets) || !aligned(pad_off) || !aligned(codes) || !aligned(scales))
    return MOE_ERR_ALIGN;
  hipError_t e = launch_pad_offsets(offsets, E, pad_off, stream);
  if (e == hipSuccess)
    e = launch_mx_quant_tokens_t(static_cast<const bf16_t*>(src), cols, nullptr, 1, offsets, pad_off, E, capacity,
                                 codes, scales, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

size_t moe_mxfp8_grouped_capacity(int32_t rows, int32_t E) {
  if (rows <= 0 || E <= 0) return 0;
  return mx_token_capacity((size_t)rows, E);
}

int32_t moe_wgrad_chunk_rows(void) { return WG_KC; }

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer argument";
    case MOE_ERR_DIMS: return "invalid dimensions";
    case MOE_ERR_UNSUPPORTED: return "unsupported mode or shape";
    case MOE_ERR_ALIGN: return "device pointer not 256-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
