// Internal declarations shared by the HIP translation units of the MoE layer
// library (kernels and the C-ABI layer).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace moe {

// ---------------------------------------------------------------------------
// Element types.  bf16 values travel as raw 16-bit patterns.
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// Round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
// Two floats -> packed pair of bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct ElemTraits<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// ---------------------------------------------------------------------------
// SwiGLU and its derivative, fp32.
//   A = SiLU(g1) * g3,  SiLU(z) = z * sigmoid(z)
//   dg1 = dA * g3 * s * (1 + g1 (1 - s)),  dg3 = dA * SiLU(g1)
// ---------------------------------------------------------------------------
// logistic sigmoid; the reciprocal is the hardware one (1 ulp), not an IEEE division
__device__ __forceinline__ float sigmoid_f32(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ---------------------------------------------------------------------------
// Problem description handed to every GEMM launcher.
// ---------------------------------------------------------------------------
struct LayerArgs {
  int T, H, I, E, k, M;
  // routing (device)
  const int32_t* offsets;         // [E+1]
  const int32_t* s2f;             // [M]
  const int32_t* f2s;             // [M]
  const float* gate;              // [T*k] flat
  // tile table for row-ragged GEMMs (device, written by build_tile_table)
  const int32_t* tile_expert;     // [max_tiles]
  const int32_t* tile_row0;       // [max_tiles]
  const int32_t* expert_tile0;    // [E+1] first row tile of each expert
  // weight-gradient work list (see WgradList) and the partial slots of split experts
  const int32_t* wg_order;        // [E]   expert of each rank (decreasing row count)
  const int32_t* wg_cstart;       // [E+1] first chunk of each rank; wg_cstart[E] = chunks
  const int32_t* wg_slot0;        // [E]   first partial slot of each rank
  const int32_t* wg_xq;           // [8 * cap] the chunks of each XCD's queue (WgradList::xq)
  float* wpart13;                 // [slots, 2I, H] fp32 partial dW13 of chunks c > 0
  float* wpart2;                  // [slots, H, I]  fp32 partial dW2
  // inputs
  const void* x;                  // [T,H]
  const void* w13;                // [E,2I,H]
  const void* w2;                 // [E,H,I]
  const void* dy;                 // [T,H]
  // forward intermediates / outputs
  int g13_f32;                    // G13 stored in fp32 (the MXFP8 backward) instead of the activation type
  void* G13;                      // [M,2I]  (saved; null when the forward keeps no state)
  void* A;                        // [M,I]   (null in the checkpointing recompute and in mxfp8 mode)
  uint8_t* q_a;                   // mxfp8 mode: MXFP8 codes of A [M,I] (written by the GEMM W13 epilogue;
                                  //   null in the checkpointing recompute, which runs no GEMM W2)
  uint8_t* q_sa;                  //   and their scales [M,I/32]
  void* O;                        // [M,H]
  // backward intermediates / outputs (fp32 in fp8_bwd mode)
  void* dG13;                     // [M,2I]
  void* Ag;                       // [M,I]   gate * A
  void* dXp;                      // [M,H]
  float* dgate_part;              // [n_parts, M]
  float* dw13;                    // [E,2I,H]
  int wgrad_acc;                  // weight gradients are added to dw13 / dw2 (accumulate-into)
  float* dw2;                     // [E,H,I]
};

// MXFP8 operands of the backward GEMMs (fp8_bwd mode).  Every operand is
// stored K-contiguous: codes [rows][K] (E4M3FN bytes) and scales [rows][K/32]
// (E8M0 bytes), K = the GEMM's reduction dimension.  The token-K operands of
// the weight gradients are transposed copies whose K is the padded token
// order: expert e's rows start at pad_off[e], a multiple of MX_KTILE, and the
// gap up to the next expert holds zero codes.
constexpr int MX_KTILE = 128;   // K elements per tile of the MXFP8 GEMMs (one scaled MFMA step)
struct Mx8Args {
  const int32_t* pad_off;       // [E+1] padded token offsets (multiples of MX_KTILE)
  int Mp;                       // padded token capacity (row length of the token-K operands)
  const uint8_t *qdy, *sdy;     // [T][H]      dY rows, K = H
  const uint8_t *qw2t, *sw2t;   // [E][I][H]   W2 transposed, K = H
  const uint8_t *qdg, *sdg;     // [M][2I]     dG13 rows, K = 2I
  const uint8_t *qw13t, *sw13t; // [E][H][2I]  W13 transposed, K = 2I
  const uint8_t *qdyt, *sdyt;   // [H][Mp]     gathered dY, K = tokens
  const uint8_t *qagt, *sagt;   // [I][Mp]     gate * A, K = tokens
  const uint8_t *qdgt, *sdgt;   // [2I][Mp]    dG13, K = tokens
  const uint8_t *qxt, *sxt;     // [H][Mp]     gathered x, K = tokens
  // mxfp8 forward
  const uint8_t *qx, *sx;       // [T][H]      x rows, K = H
  const uint8_t *qw13, *sw13;   // [E][2I][H]  W13 rows, K = H
  const uint8_t *qa, *sa;       // [M][I]      A rows, K = I
  const uint8_t *qw2, *sw2;     // [E][H][I]   W2 rows, K = I
};
// Padded token capacity: every expert rounds its count up to MX_KTILE.
inline size_t mx_token_capacity(size_t M, int E) {
  return (M + MX_KTILE - 1) / MX_KTILE * MX_KTILE + (size_t)E * MX_KTILE;
}

// Number of M tiles of height bm over all experts is at most this bound.
inline int max_row_tiles(int M, int E, int bm) { return (M + bm - 1) / bm + E; }

// GEMM kinds of the layer.
enum GemmKind {
  KIND_FWD1 = 0,   // G13 = Xp W13^T, SwiGLU epilogue -> G13 (saved), A
  KIND_FWD2 = 1,   // O = A W2^T
  KIND_DGRAD2 = 2, // dA' = dYp W2; epilogue: dgate partials, Ag, dSwiGLU -> dG13
  KIND_DGRAD1 = 3, // dXp = dG13 W13
  KIND_WGRAD2 = 4, // dW2[e] = dYp^T Ag     (K = rows of e)
  KIND_WGRAD1 = 5  // dW13[e] = dG13^T Xp   (K = rows of e)
};

// ---------------------------------------------------------------------------
// Kernel launch through hipLaunchKernel: returns the status of this launch
// itself, never an error left behind by an earlier, unrelated HIP call (and
// leaves the caller's last-error state alone when the launch succeeds).
// ---------------------------------------------------------------------------
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                                A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<std::remove_cv_t<std::remove_reference_t<P>>...> vals(std::forward<A>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {const_cast<void*>(static_cast<const void*>(&v))...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, s);
      },
      vals);
}

// ---------------------------------------------------------------------------
// Launchers (each returns the status of its own launches; a launcher with
// several kernels stops at the first failure).
// ---------------------------------------------------------------------------
// routing
// router projection (router.hip): logits = x W_r^T; backward: dx += dlogits W_r, dW_r = dlogits^T x
hipError_t launch_router_logits(const bf16_t* x, const bf16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t s);
hipError_t launch_router_project_bwd(const float* dlogits, const int32_t* topk_idx, const int32_t* offsets,
                                     const int32_t* s2f, const bf16_t* x, const bf16_t* wr, int T, int H, int E,
                                     int k, bf16_t* dx, float* dwr, hipStream_t s);
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* topk_idx, float* gate,
                        int32_t* counts, int32_t* offsets, int32_t* s2f, int32_t* f2s,
                        int32_t* ws_partials, int32_t* ws_bases, hipStream_t s);
int route_num_blocks(int M);   // blocks of the histogram / scatter passes
// Library-held routing scratch of moe_route_noalloc (a static device array,
// one per GPU): its size, and this device's address of it (looked up once per
// device, on the first call with that device current).
constexpr size_t ROUTE_SCRATCH_BYTES = (size_t)2 << 20;
hipError_t route_scratch_ptr(void** ptr);

// Rows per weight-gradient chunk: an expert with more rows is split along K
// (its rows) into chunks of WG_KC rows (a multiple of the 128-row MXFP8 K tile
// and of every bf16 K tile), whose fp32 results are summed in chunk order.
// 8192 rows: with the chunks dealt to balanced XCD queues, 8192- and
// 12288-row chunks measured 9 % faster than 4096 over the skewed layer's
// weight gradients and their ordered reduction (less partial-slot traffic),
// 16384 slower (too coarse for the XCD queues).
#ifndef MOE_WG_KC
#define MOE_WG_KC 8192
#endif
constexpr int WG_KC = MOE_WG_KC;
// Fixed cost of a weight-gradient tile in rows of K (its fp32 output write
// and pipeline fill), used when the chunks are dealt to the XCD queues.
constexpr int WG_BETA = 384;
struct WgradList {              // device tables written by the backward's tile-table kernel
  int32_t* order;               // [E]   expert of each rank, by decreasing row count (ties: index)
  int32_t* cstart;              // [E+1] first chunk of each rank (exclusive prefix of the chunk counts)
  int32_t* slot0;               // [E]   first partial slot of each rank (prefix of chunks - 1)
  int32_t* xq;                  // [8 * cap] chunks of XCD x's queue at xq[x * cap + q], cap = ceil(chunks / 8),
                                //           -1 past the queue's end
};
// partial slots the split experts can need: sum over experts of (chunks - 1) <= M / WG_KC
inline size_t wgrad_max_slots(size_t M) { return M / WG_KC; }
// upper bound of the number of chunks: E + M / WG_KC
inline int wgrad_max_chunks(int M, int E) { return E + M / WG_KC; }
// entries of the XCD queue table for max_chunks chunks
inline int wgrad_queue_slots(int max_chunks) { return 8 * ((max_chunks + 7) / 8); }

hipError_t launch_tile_table(const int32_t* offsets, int E, int bm, int max_tiles,
                             int32_t* tile_expert, int32_t* tile_row0, int32_t* expert_tile0, WgradList wg, hipStream_t s);
// dW[e] += the partial slots of each split expert, in chunk order (both matrices)
hipError_t launch_wgrad_reduce(const LayerArgs& a, hipStream_t s);

// combine / unpermute-reduce (fp32 accumulate in slot order)
template <typename T>
hipError_t launch_combine(const T* rows, const int32_t* f2s, const float* gate, int Tn, int k, int H,
                          T* out, hipStream_t s);
// router backward: dgate from per-N-tile partials, then the logit gradient
hipError_t launch_router_bwd(const float* dgate_part, int n_parts, const int32_t* f2s,
                             const float* gate, const int32_t* topk_idx, int Tn, int k, int E, int M,
                             float* dgate, float* dlogits, hipStream_t s);

// GEMMs
hipError_t launch_gemm_bf16(GemmKind kind, const LayerArgs& a, hipStream_t s);
hipError_t launch_gemm_fp32(GemmKind kind, const LayerArgs& a, hipStream_t s);

// MXFP8 GEMMs (every kind)
hipError_t launch_gemm_mx8(GemmKind kind, const LayerArgs& a, const Mx8Args& q, hipStream_t s);
int mx8_fwd_row_tile_m();   // token rows per tile of the MXFP8 forward GEMMs
int mx8_row_tile_m();       // token rows per tile of the MXFP8 dgrad GEMMs
int mx8_dgrad2_tile_n();    // columns per tile of the MXFP8 dgrad of W2

// MXFP8 quantisers (E4M3FN codes + E8M0 scales per 32 elements, round to
// nearest even, saturating).  Layouts as in Mx8Args.
//   rows:      src [R][K] (row src_row(r) = s2f ? s2f[r]/k : r) -> codes [R][K], scales [R][K/32]
//   cols_t:    per expert, src [Kd][N] -> codes [N][Kd], scales [N][Kd/32]   (Kd % MX_KTILE == 0)
//   tokens_t:  src rows r of the expert-sorted order (gathered as above) of a
//              [.][F] matrix -> codes [F][Mp], scales [F][Mp/32], expert e's
//              rows at pad_off[e] .. (zero-padded to the next multiple of MX_KTILE)
template <typename T>   // instantiated for T = bf16_t
hipError_t launch_mx_quant_rows(const T* src, int R, int K, const int32_t* s2f, int k, uint8_t* codes,
                                uint8_t* scales, hipStream_t s);
hipError_t launch_mx_quant_cols_t(const bf16_t* src, int E, int Kd, int N, uint8_t* codes, uint8_t* scales,
                                  hipStream_t s);
// Both MXFP8 copies of dense weights [E][Kd][N] from one read: transposed
// ([E][N][Kd], blocks of 32 along Kd, as launch_mx_quant_cols_t) and row-wise
// ([E*Kd][N], blocks of 32 along N, as launch_mx_quant_rows).  N % 64 == 0,
// Kd % 128 == 0.
hipError_t launch_mx_quant_both(const bf16_t* src, int E, int Kd, int N, uint8_t* codes_t, uint8_t* scales_t,
                                uint8_t* codes_r, uint8_t* scales_r, hipStream_t s);
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* pad_off, hipStream_t s);
template <typename T>   // instantiated for T = bf16_t
hipError_t launch_mx_quant_tokens_t(const T* src, int F, const int32_t* s2f, int k, const int32_t* offsets,
                                    const int32_t* pad_off, int E, int Mp, uint8_t* codes, uint8_t* scales,
                                    hipStream_t s);

// tiling the API layer needs for workspace sizing and the tile table
int bf16_fwd_row_tile_m();  // token rows per tile of the bf16 forward GEMMs
bool bf16_dgrad_long(int H, int I);  // the bf16 dgrad GEMMs take their long-K tiles
int bf16_row_tile_m(int H, int I);   // token rows per tile of the bf16 dgrad GEMMs
int bf16_dgrad2_tile_n();   // columns per tile of the bf16 dgrad of W2
constexpr int FP32_BM = 64;
constexpr int FP32_BN = 64;
// mode: 0 fp32, 1 bf16, 2 mxfp8, 3 fp8_bwd (the public moe_mode values)
inline bool mx8_forward(int mode) { return mode == 2; }
inline bool mx8_backward(int mode) { return mode == 2 || mode == 3; }
// Weight-gradient tile of virtual block vb (the block index of a grid with
// one block per tile): block b goes to XCD x = b % 8 (round-robin dispatch),
// and XCD x takes the chunks of its queue (the tile-table kernel deals the
// chunks, in work-list order, to the least loaded queue with room; every queue
// holds at most cap = ceil(chunks / 8)) in order, each as per_e consecutive
// tiles, which share the chunk's rows in that XCD's L2.
// Gives the expert e, its rows [r0, r1) (expert-local), the partial slot (-1
// for chunk 0, which writes dW[e]) and the tile t; false past the queue's end.
__device__ __forceinline__ bool decode_wgrad_tile(const LayerArgs& a, int vb, int per_e, int& e, int& r0, int& r1,
                                                  int& slot, int& t) {
  const int x = vb % 8, j = vb / 8;
  const int q = j / per_e;
  const int cap = (a.wg_cstart[a.E] + 7) / 8;
  if (q >= cap) return false;
  const int item = a.wg_xq[x * cap + q];
  if (item < 0) return false;
  int lo = 0, hi = a.E - 1;               // rank with cstart[rank] <= item (cstart strictly increasing)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.wg_cstart[mid] <= item) lo = mid; else hi = mid - 1;
  }
  e = a.wg_order[lo];
  const int c = item - a.wg_cstart[lo];
  const int cnt = a.offsets[e + 1] - a.offsets[e];
  r0 = c * WG_KC;
  r1 = min(cnt, r0 + WG_KC);
  slot = c == 0 ? -1 : a.wg_slot0[lo] + c - 1;
  t = j % per_e;
  return true;
}
inline int wgrad_grid(int max_chunks, int per_e) { return 8 * ((max_chunks + 7) / 8) * per_e; }
// Blocks of a persistent GEMM grid: per_cu resident blocks on every compute
// unit of the current device, a multiple of the 8 XCDs (block b runs on XCD
// b % 8, so a block keeps its XCD from one virtual block to the next).
int resident_blocks(int per_cu);

inline int fwd_row_tile_m(int mode) {
  return mode == 0 ? FP32_BM : mx8_forward(mode) ? mx8_fwd_row_tile_m() : bf16_fwd_row_tile_m();
}
inline int bwd_row_tile_m(int mode, int H, int I) {
  return mode == 0 ? FP32_BM : mx8_backward(mode) ? mx8_row_tile_m() : bf16_row_tile_m(H, I);
}
inline int dgrad2_parts(int mode, int I) {
  // N tiles of the dgrad of W2 (N = I): one gate-gradient partial per tile
  const int bn = mode == 0 ? FP32_BN : mx8_backward(mode) ? mx8_dgrad2_tile_n() : bf16_dgrad2_tile_n();
  return (I + bn - 1) / bn;
}

}  // namespace moe
