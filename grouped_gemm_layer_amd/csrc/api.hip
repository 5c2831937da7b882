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

struct Sizes {
  size_t route_ws, saved, fwd_ws, bwd_ws;
  // carving offsets
  size_t r_partials, r_bases;
  size_t f_tile_e, f_tile_r, f_tile_x, f_A, f_O;
  size_t b_tile_e, b_tile_r, b_tile_x, b_dG13, b_Ag, b_dXp, b_part;
};

moe_status check_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->T <= 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->k <= 0 || d->k > d->E) return MOE_ERR_DIMS;
  if ((int64_t)d->T * d->k > INT32_MAX) return MOE_ERR_DIMS;
  if ((int64_t)d->E * 2 * d->I * d->H > ((int64_t)1 << 40)) return MOE_ERR_DIMS;
  if (d->mode != MOE_MODE_FP32 && d->mode != MOE_MODE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->H % 64 != 0 || d->I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->E > 512 || d->k > 32) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Sizes compute_sizes(const moe_dims* d) {
  Sizes s{};
  const size_t M = (size_t)d->T * d->k;
  const size_t es = (d->mode == MOE_MODE_FP32) ? 4 : 2;
  const bool bf16 = d->mode != MOE_MODE_FP32;
  const int bm = row_tile_m(bf16);
  const size_t max_tiles = (size_t)max_row_tiles((int)M, d->E, bm);
  const size_t nblk = (size_t)route_num_blocks((int)M);
  size_t o = 0;
  s.r_partials = o; o += align_up(nblk * d->E * 4);
  s.r_bases = o;    o += align_up(nblk * d->E * 4);
  s.route_ws = o;
  s.saved = align_up(M * 2 * d->I * es);
  o = 0;
  s.f_tile_e = o; o += align_up(max_tiles * 4);
  s.f_tile_r = o; o += align_up(max_tiles * 4);
  s.f_tile_x = o; o += align_up(((size_t)d->E + 1) * 4);
  s.f_A = o;      o += align_up(M * d->I * es);
  s.f_O = o;      o += align_up(M * d->H * es);
  s.fwd_ws = o;
  o = 0;
  s.b_tile_e = o; o += align_up(max_tiles * 4);
  s.b_tile_r = o; o += align_up(max_tiles * 4);
  s.b_tile_x = o; o += align_up(((size_t)d->E + 1) * 4);
  s.b_dG13 = o;   o += align_up(M * 2 * d->I * es);
  s.b_Ag = o;     o += align_up(M * d->I * es);
  s.b_dXp = o;    o += align_up(M * d->H * es);
  s.b_part = o;   o += align_up((size_t)dgrad2_parts(bf16, d->I) * M * 4);
  s.bwd_ws = o;
  return s;
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

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

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
constexpr int kBackwardKernels = 7;   // tile table, dgrad W2 + dSwiGLU, dgrad W13, unpermute, router, wgrad W2, wgrad W13

moe_status forward_impl(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                        const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                        hipStream_t stream, Marks mk);
moe_status backward_impl(const moe_dims* dims, const void* dy, const void* x, const void* w13, const void* w2,
                         const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                         float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream, Marks mk);

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

}  // extern "C"

namespace {

moe_status forward_impl(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                        const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                        hipStream_t stream, Marks mk) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  if (!x || !w13 || !w2 || !y || !saved || !ws) return MOE_ERR_NULL;
  if (!aligned(x) || !aligned(w13) || !aligned(w2) || !aligned(y) || !aligned(saved) || !aligned(ws))
    return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  if (ws_bytes < s.fwd_ws) return MOE_ERR_WORKSPACE;
  const bool bf16 = dims->mode != MOE_MODE_FP32;
  LayerArgs a = base_args(dims, routing);
  a.x = x; a.w13 = w13; a.w2 = w2;
  a.G13 = saved;
  a.A = at(ws, s.f_A);
  a.O = at(ws, s.f_O);
  int32_t* te = reinterpret_cast<int32_t*>(at(ws, s.f_tile_e));
  int32_t* tr = reinterpret_cast<int32_t*>(at(ws, s.f_tile_r));
  int32_t* tx = reinterpret_cast<int32_t*>(at(ws, s.f_tile_x));
  a.tile_expert = te; a.tile_row0 = tr; a.expert_tile0 = tx;
  const int bm = row_tile_m(bf16);
  hipError_t e = mk.mark();
  if (e == hipSuccess) e = launch_tile_table(routing->offsets, dims->E, bm, max_row_tiles(a.M, a.E, bm), te, tr, tx, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) e = gemm(bf16, KIND_FWD1, a, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) e = gemm(bf16, KIND_FWD2, a, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) {
    if (bf16)
      e = launch_combine<bf16_t>(static_cast<const bf16_t*>(a.O), a.f2s, a.gate, a.T, a.k, a.H,
                                 static_cast<bf16_t*>(y), stream);
    else
      e = launch_combine<float>(static_cast<const float*>(a.O), a.f2s, a.gate, a.T, a.k, a.H,
                                static_cast<float*>(y), stream);
  }
  if (e == hipSuccess) e = mk.mark();
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status backward_impl(const moe_dims* dims, const void* dy, const void* x, const void* w13, const void* w2,
                         const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                         float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream, Marks mk) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  if (!dy || !x || !w13 || !w2 || !saved || !dx || !dw13 || !dw2 || !dgate || !ws) return MOE_ERR_NULL;
  if (!aligned(dy) || !aligned(x) || !aligned(w13) || !aligned(w2) || !aligned(saved) || !aligned(dx) ||
      !aligned(dw13) || !aligned(dw2) || !aligned(dgate) || !aligned(ws) || (dlogits && !aligned(dlogits)))
    return MOE_ERR_ALIGN;
  const Sizes s = compute_sizes(dims);
  if (ws_bytes < s.bwd_ws) return MOE_ERR_WORKSPACE;
  const bool bf16 = dims->mode != MOE_MODE_FP32;
  LayerArgs a = base_args(dims, routing);
  a.x = x; a.w13 = w13; a.w2 = w2; a.dy = dy;
  a.G13 = const_cast<void*>(saved);
  a.dG13 = at(ws, s.b_dG13);
  a.Ag = at(ws, s.b_Ag);
  a.dXp = at(ws, s.b_dXp);
  a.dgate_part = reinterpret_cast<float*>(at(ws, s.b_part));
  a.dw13 = dw13;
  a.dw2 = dw2;
  int32_t* te = reinterpret_cast<int32_t*>(at(ws, s.b_tile_e));
  int32_t* tr = reinterpret_cast<int32_t*>(at(ws, s.b_tile_r));
  int32_t* tx = reinterpret_cast<int32_t*>(at(ws, s.b_tile_x));
  a.tile_expert = te; a.tile_row0 = tr; a.expert_tile0 = tx;
  const int bm = row_tile_m(bf16);
  // activation-gradient chain first; the weight gradients do not feed it
  hipError_t e = mk.mark();
  if (e == hipSuccess) e = launch_tile_table(routing->offsets, dims->E, bm, max_row_tiles(a.M, a.E, bm), te, tr, tx, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) e = gemm(bf16, KIND_DGRAD2, a, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) e = gemm(bf16, KIND_DGRAD1, a, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) {
    if (bf16)
      e = launch_combine<bf16_t>(static_cast<const bf16_t*>(a.dXp), a.f2s, nullptr, a.T, a.k, a.H,
                                 static_cast<bf16_t*>(dx), stream);
    else
      e = launch_combine<float>(static_cast<const float*>(a.dXp), a.f2s, nullptr, a.T, a.k, a.H,
                                static_cast<float*>(dx), stream);
  }
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess)
    e = launch_router_bwd(a.dgate_part, dgrad2_parts(bf16, a.I), a.f2s, a.gate, routing->topk_idx, a.T, a.k,
                          a.E, a.M, dgate, dlogits, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) e = gemm(bf16, KIND_WGRAD2, a, stream);
  if (e == hipSuccess) e = mk.mark();
  if (e == hipSuccess) e = gemm(bf16, KIND_WGRAD1, a, stream);
  if (e == hipSuccess) e = mk.mark();
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                       const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return forward_impl(dims, x, w13, w2, routing, y, saved, ws, ws_bytes, stream, Marks{nullptr, 0, 0, stream});
}

moe_status moe_backward(const moe_dims* dims, const void* dy, const void* x, const void* w13, const void* w2,
                        const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                        float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream) {
  return backward_impl(dims, dy, x, w13, w2, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes, stream,
                       Marks{nullptr, 0, 0, stream});
}

int moe_num_kernels(int which) {
  return which == 0 ? kRouteKernels : which == 1 ? kForwardKernels : which == 2 ? kBackwardKernels : -1;
}

moe_status moe_forward_timed(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                             const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                             hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!events) return MOE_ERR_NULL;
  if (n_events < kForwardKernels + 1) return MOE_ERR_DIMS;
  return forward_impl(dims, x, w13, w2, routing, y, saved, ws, ws_bytes, stream,
                      Marks{events, n_events, 0, stream});
}

moe_status moe_backward_timed(const moe_dims* dims, const void* dy, const void* x, const void* w13,
                              const void* w2, const moe_routing* routing, const void* saved, void* dx,
                              float* dw13, float* dw2, float* dgate, float* dlogits, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!events) return MOE_ERR_NULL;
  if (n_events < kBackwardKernels + 1) return MOE_ERR_DIMS;
  return backward_impl(dims, dy, x, w13, w2, routing, saved, dx, dw13, dw2, dgate, dlogits, ws, ws_bytes, stream,
                       Marks{events, n_events, 0, stream});
}

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
