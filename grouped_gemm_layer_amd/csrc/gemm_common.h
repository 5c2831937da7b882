// Shared pieces of the grouped-GEMM kernels (bf16 and MXFP8): tile
// configuration and the fused epilogues of the six GEMM kinds.  Internal.
#pragma once

#include "moe_internal.h"
#include "mx_codec.h"

namespace moe {
namespace gg {

constexpr int NXCD = 8;   // XCDs per MI355X; blocks are dealt to them round-robin
constexpr uint32_t OOB = 0x80000000u;   // buffer offset that reads as zeros

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // one 16-byte chunk


// Raw buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer loads straight into LDS: lane l writes LDS bytes [m0 + W l, +W) for
// W = 16 (dma16) or 4 (dma4).  Issued as inline assembly so that the compiler
// neither tracks nor waits on them; completion is awaited explicitly
// (vm_wait) before the barrier that publishes a stage.  An offset past the
// buffer's end stores zeros.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t lds_m0) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(byte_off), "s"(r), "s"(lds_m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t lds_m0) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(byte_off), "s"(r), "s"(lds_m0) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Logical tile L of a row-ragged GEMM -> (expert, first row, column tile).
// Order: expert-major; inside an expert, groups of gn column tiles, and inside
// a group all of the expert's row tiles with the gn columns fastest, so that
// about one XCD's worth of concurrent blocks (`group` blocks) shares the same
// token rows and weight rows.  Returns false for an unused tile.
struct RowTile { int e, m0, mlim, nt; };
__device__ __forceinline__ bool decode_row_tile(const LayerArgs& a, int L, int n_tiles, int group, RowTile& t) {
  const int e = a.tile_expert[L / n_tiles];
  if (e < 0) return false;
  const int t0 = a.expert_tile0[e];
  const int me = a.expert_tile0[e + 1] - t0;            // row tiles of this expert
  const int local = L - t0 * n_tiles;
  const int gn = max(1, min(n_tiles, group / me));
  const int ng = local / (me * gn);
  const int gs = min(gn, n_tiles - ng * gn);
  const int rem = local - ng * me * gn;
  t.e = e;
  t.nt = ng * gn + rem % gs;
  t.m0 = a.tile_row0[t0 + rem / gs];
  t.mlim = a.offsets[e + 1];
  return true;
}

template <int BM_, int BN_, int WGM_, int WGN_, int WPE_, int ST_, int BK_ = 64, int GD_ = 1, int PIPE_ = 0,
          int PERSIST_ = 0>
struct TileCfg {
  // grid: 0 = one block per tile; 1 = persistent, the resident blocks loop
  // over the tiles in the same order
  static constexpr int PERSIST = PERSIST_;
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_;
  // main loop: 0 = every wave reads a whole K tile's fragments between two
  // barriers, then runs its MFMAs; 1 = software pipeline, the fragments of the
  // next 32-wide K step are read while the MFMAs of the current one run (one
  // barrier per K tile); 2 = ping-pong between the two wave rows (row kinds
  // of the bf16 kernel: one row reads a K tile while the other multiplies)
  static constexpr int PIPE = PIPE_;
  static constexpr int WPE = WPE_;      // waves per SIMD the register allocation must allow
  static constexpr int STAGES = ST_;    // LDS stages in flight (>= 2)
  static constexpr int NW = WGM * WGN, NTHR = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 16, FN = WN / 16;
  // 1 KiB LDS DMA instructions per wave per K tile, A and B operands
  // (bf16 operands: BK elements = 2*BK bytes per row)
  static constexpr int DA = BM * BK * 2 / 1024 / NW, DB = BN * BK * 2 / 1024 / NW;
  // tile groups that share operands: blocks resident on one XCD at a time,
  // divided by GD (smaller groups measured faster for the forward kinds)
  static constexpr int GROUP = 32 * (4 * WPE) / NW / GD_;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(DA * NW * 1024 == BM * BK * 2 && DB * NW * 1024 == BN * BK * 2, "tiles must split into 1 KiB DMA rows");
  static constexpr int SMEM_BYTES = STAGES * (BM + BN) * BK * 2;   // operand LDS of the kernel
  static_assert(STAGES >= 2, "need at least two LDS stages");
  static_assert(BK == 32 || BK == 64, "K tile of 32 or 64");
};

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2_t pack4(float a, float b, float c, float d) {
  return u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// Stores of GEMM outputs.  NT = non-temporal: used for the weight
// gradients, whose LDS-staged stores write whole lines that this launch
// never reads again (measured faster); the row kinds' 8- and 16-byte stores
// need the L2 to combine them into lines (non-temporal is slower there).
template <bool NT = false, class V, class P>
__device__ __forceinline__ void st_out(P* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else *reinterpret_cast<V*>(p) = v;
}

// Cross-lane reductions without LDS traffic (DPP and the gfx950 row swaps).
// The maxima are taken over the bit patterns of non-negative floats, which
// order like the values.
// maximum over the 16 lanes of each row (lanes 16r .. 16r+15)
__device__ __forceinline__ uint32_t umax_row16(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  return v;
}
// umax_row16 over a whole array, one DPP step at a time across all elements
// (independent chains back to back need no wait states between steps)
template <int CTRL, int N0, int N1, int N2>
__device__ __forceinline__ void umax_dpp_step(uint32_t (&v)[N0][N1][N2]) {
#pragma unroll
  for (int a = 0; a < N0; ++a)
#pragma unroll
    for (int b = 0; b < N1; ++b)
#pragma unroll
      for (int c = 0; c < N2; ++c)
        v[a][b][c] = max(v[a][b][c], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[a][b][c], CTRL, 0xF, 0xF, false));
}
template <int N0, int N1, int N2>
__device__ __forceinline__ void row16_umax_steps(uint32_t (&v)[N0][N1][N2]) {
  umax_dpp_step<0xB1>(v);    // quad_perm 1,0,3,2
  umax_dpp_step<0x4E>(v);    // quad_perm 2,3,0,1
  umax_dpp_step<0x141>(v);   // row_half_mirror
  umax_dpp_step<0x140>(v);   // row_mirror
}
// maximum over the lanes l, l^16, l^32, l^48
__device__ __forceinline__ uint32_t umax_rows4(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)r[0], (uint32_t)r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}
// sum over the lanes l, l^16, l^32, l^48 (every lane gets the same value)
__device__ __forceinline__ float fsum_rows4(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
// sum over the 32 lanes of each half wave (every lane gets the same value)
__device__ __forceinline__ float fsum_lanes32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// Gate-gradient partials of one tile: lanes sharing a row, then the WGN waves
// of a row block, in a fixed order.  `s_part` holds WGN * BM floats of LDS.
template <class C>
__device__ __forceinline__ void dgate_partials(const LayerArgs& a, float (&psum)[C::FM], float* s_part, int tid,
                                               int lane, int wm, int wn, int m0, int mlim, int n0) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i) psum[i] = fsum_rows4(psum[i]);
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) s_part[wn * C::BM + wm * C::WM + 16 * i + lane] = psum[i];
  }
  __syncthreads();
  for (int ml = tid; ml < C::BM; ml += C::NTHR) {
    const int m = m0 + ml;
    if (m < mlim) {
      float p = 0.f;
#pragma unroll
      for (int w = 0; w < C::WGN; ++w) p += s_part[w * C::BM + ml];
      a.dgate_part[(size_t)(n0 / C::BN) * a.M + m] = p;
    }
  }
}

// Writes one output tile of the row kinds through LDS, so that every store
// instruction covers whole rows: a lane holds 4 consecutive columns of 16
// rows (pieces spread over 16 lines), the copy-out stores 16 bytes per lane
// along rows.  `val(i, j)` returns the 4 values of the wave's row block i and
// fragment j (0 <= j < FJ), tile columns wn*16*FJ + 16 j + 4*(lane/16) .. +3,
// as 4 packed bf16 (u32x2_t) or 4 floats (f32x4_t).  Row m, tile column t
// goes to out[m * ld + c0 + t] for m < mlim and c0 + t < clim (clim a
// multiple of the 16-byte chunk).  The tile passes in chunks of CH rows when
// it exceeds the operand LDS.  The caller has freed the LDS (barrier after
// the main loop); the function ends with a barrier, so the LDS may be
// reused after it.
template <class C, int FJ, class T, class Val>
__device__ __forceinline__ void staged_store(void* smem, Val&& val, T* out, size_t ld, int m0, int mlim, int c0,
                                             int clim, int tid, int lane, int wm, int wn) {
  using V = decltype(val(0, 0));
  constexpr int BM = C::BM, WM = C::WM, FM = C::FM, NTHR = C::NTHR;
  constexpr int VB = (int)sizeof(V);                      // bytes of 4 values
  static_assert(VB == 4 * (int)sizeof(T), "values match the output type");
  constexpr int TW = C::WGN * 16 * FJ;                    // tile width (elements)
  constexpr int RB = TW * (VB / 4);                       // bytes per tile row
  constexpr int NQ = RB / 16, EQ = 16 / (VB / 4);         // 16-byte chunks per row, elements per chunk
  constexpr int CH0 = C::SMEM_BYTES / RB;
  constexpr int CH = CH0 >= BM ? BM : CH0 >= 64 ? 64 : CH0 >= 32 ? 32 : 16;
  static_assert(CH * RB <= C::SMEM_BYTES && BM % CH == 0 && CH % 16 == 0 && WM % 16 == 0,
                "row chunk must fit in the operand LDS");
  uint8_t* s = static_cast<uint8_t*>(smem);
  const int mrow = lane & 15, ncol = 4 * (lane >> 4);
  auto off = [&](int row, int q) { return row * RB + ((q ^ (row % NQ)) << 4); };
#pragma unroll
  for (int ch = 0; ch < BM / CH; ++ch) {
    if (ch > 0) __syncthreads();                          // the previous chunk has been read out
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if ((wm * WM + 16 * i) / CH != ch) continue;        // a 16-row block lies in one chunk
      const int row = wm * WM + 16 * i + mrow - ch * CH;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int byte = (wn * 16 * FJ + 16 * j + ncol) * (VB / 4);
        *reinterpret_cast<V*>(s + off(row, byte >> 4) + (byte & 15)) = val(i, j);
      }
    }
    __syncthreads();
    for (int c = tid; c < CH * NQ; c += NTHR) {
      const int row = c / NQ, q = c % NQ;
      const int m = m0 + ch * CH + row, n = c0 + EQ * q;
      if (m < mlim && n < clim)
        *reinterpret_cast<u32x4_t*>(out + (size_t)m * ld + n) = *reinterpret_cast<const u32x4_t*>(s + off(row, q));
    }
  }
  __syncthreads();
}

// Output of a weight-gradient tile: dW[e] for the first chunk of expert e,
// else the chunk's partial slot (added to dW[e] in chunk order afterwards).
// With accumulate-into (a.wgrad_acc) only dW[e] adds the caller's value.
template <int KIND>
__device__ __forceinline__ float* wgrad_out(const LayerArgs& a, int e, int slot) {
  const size_t n = KIND == KIND_WGRAD2 ? (size_t)a.H * a.I : (size_t)2 * a.I * a.H;
  float* base = slot < 0 ? (KIND == KIND_WGRAD2 ? a.dw2 : a.dw13) : (KIND == KIND_WGRAD2 ? a.wpart2 : a.wpart13);
  return base + (size_t)(slot < 0 ? e : slot) * n;
}

// Epilogue of one output tile.  acc[i][j][v] holds C[m][n] for
//   m = m0 + wm*WM + 16 i + lane%16,  n = n0 + wn*WN + 16 j + 4*(lane/16) + v
// (for the SwiGLU kind the first FN/2 column blocks are G1 and the rest the
// matching G3 columns).  `smem` is the kernel's operand LDS, free by now.
// MX8: epilogue of the MXFP8 kernels -- GEMM W13 + SwiGLU writes A as the
// MXFP8 operand of GEMM W2 (the dgrad of W2 has dgrad2_epilogue_mx8).
template <int KIND, class C, bool MX8 = false>
__device__ __forceinline__ void gemm_epilogue(const LayerArgs& a, f32x4_t (&acc)[C::FM][C::FN], void* smem,
                                              int tid, int lane, int wm, int wn, int e, int m0, int mlim,
                                              int n0, int nlim, float* wout = nullptr, bool wacc = false) {
  constexpr int BM = C::BM, BN = C::BN, NTHR = C::NTHR, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  const int H = a.H, I = a.I;
  // ---------------- epilogues ----------------
  const int mrow = lane & 15;         // row inside a 16x16 block
  const int ncol = 4 * (lane >> 4);   // first of 4 consecutive columns

  if constexpr (KIND == KIND_FWD1) {
    // the first FN/2 fragments hold G1 columns, the rest the matching G3 columns
    constexpr int FH = FN / 2;
    const int c0 = n0;
    const size_t ld13 = (size_t)2 * I;
    auto gv = [&](int i, int j) { const f32x4_t g = acc[i][j]; return pack4(g[0], g[1], g[2], g[3]); };
    auto av = [&](int i, int j) {
      const f32x4_t g1 = acc[i][j], g3 = acc[i][j + FH];
      return f32x4_t{g1[0] * sigmoid_f32(g1[0]) * g3[0], g1[1] * sigmoid_f32(g1[1]) * g3[1],
                     g1[2] * sigmoid_f32(g1[2]) * g3[2], g1[3] * sigmoid_f32(g1[3]) * g3[3]};
    };
    // G13 is the state the backward reads: none when the forward keeps nothing
    if (a.G13 == nullptr) {
    } else if (a.g13_f32) {   // saved state kept in fp32 (the MXFP8 backward quantises from it)
      float* G13 = static_cast<float*>(a.G13);
      staged_store<C, FH>(smem, [&](int i, int j) { return acc[i][j]; }, G13, ld13, m0, mlim, c0, I, tid, lane, wm, wn);
      staged_store<C, FH>(smem, [&](int i, int j) { return acc[i][j + FH]; }, G13 + I, ld13, m0, mlim, c0, I, tid,
                          lane, wm, wn);
    } else {
      bf16_t* G13 = static_cast<bf16_t*>(a.G13);
      staged_store<C, FH>(smem, gv, G13, ld13, m0, mlim, c0, I, tid, lane, wm, wn);
      staged_store<C, FH>(smem, [&](int i, int j) { return gv(i, j + FH); }, G13 + I, ld13, m0, mlim, c0, I, tid,
                          lane, wm, wn);
    }
    // A feeds only the GEMM W2: the checkpointing recompute passes no A buffer
    if constexpr (MX8) {
      if (a.q_a == nullptr) return;
      // MXFP8 operand of the GEMM W2 straight from fp32: blocks of 32 along I
      // are fragment pairs (2jb, 2jb+1); the 4 lanes sharing a row reduce the
      // block maximum with row swaps, codes leave through LDS along rows and
      // the scale byte from the lane holding the block's first columns
      static_assert(FH % 2 == 0, "a block of 32 columns = two fragments");
      const auto r_sa = make_rsrc(a.q_sa, (uint32_t)a.M * (I / 32));
      int X[FM][FH / 2];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + 16 * i + mrow;
#pragma unroll
        for (int jb = 0; jb < FH / 2; ++jb) {
          const f32x4_t v0 = av(i, 2 * jb), v1 = av(i, 2 * jb + 1);
          uint32_t amax = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) amax = max(amax, max(abs_bits(v0[v]), abs_bits(v1[v])));
          X[i][jb] = mx_scale_exp(__uint_as_float(umax_rows4(amax)));
          const int cb = c0 + wn * 16 * FH + 32 * jb;   // first column of the block
          if (ncol == 0)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(X[i][jb] + 127), r_sa,
                                                 (m < mlim && cb < I) ? (uint32_t)m * (I / 32) + cb / 32 : OOB, 0, 0);
        }
      }
      staged_store<C, FH>(smem, [&](int i, int j) { const f32x4_t v = av(i, j); return mx_pack4(v[0], v[1], v[2], v[3], X[i][j / 2]); },
                          static_cast<uint8_t*>(a.q_a), (size_t)I, m0, mlim, c0, I, tid, lane, wm, wn);
    } else if (a.A != nullptr) {
      staged_store<C, FH>(smem, [&](int i, int j) { const f32x4_t v = av(i, j); return pack4(v[0], v[1], v[2], v[3]); },
                          static_cast<bf16_t*>(a.A), (size_t)I, m0, mlim, c0, I, tid, lane, wm, wn);
    }
  } else if constexpr (KIND == KIND_FWD2 || KIND == KIND_DGRAD1) {
    bf16_t* out = static_cast<bf16_t*>(KIND == KIND_FWD2 ? a.O : a.dXp);
    staged_store<C, FN>(smem, [&](int i, int j) { const f32x4_t v = acc[i][j]; return pack4(v[0], v[1], v[2], v[3]); },
                        out, (size_t)H, m0, mlim, n0, nlim, tid, lane, wm, wn);
  } else if constexpr (KIND == KIND_DGRAD2) {
    static_assert(!MX8, "the MXFP8 kernels use dgrad2_epilogue_mx8");
    // dA' = acc passes through LDS in fp32, CH rows at a time; then each
    // thread takes 8 consecutive columns of one row: coalesced 16-byte loads
    // of G1 and G3, stores of dG1, dG3 and g*A, and the row's gate-gradient
    // partial summed over the 32 lanes that hold the row (fixed order).  All
    // gate and G13 loads of a chunk are issued before the chunk is staged, so
    // their latency overlaps the LDS transpose and each other instead of
    // stalling every row in turn.
    constexpr int NQ4 = BN / 4;                            // 16-byte fp32 chunks per row
    constexpr int TPR = BN / 8;                            // threads per row
    static_assert(TPR == 32 && NTHR % TPR == 0, "one row per half wave");
    constexpr int CH0 = C::SMEM_BYTES / (BN * 4);
    constexpr int CH = CH0 >= BM ? BM : CH0 >= 64 ? 64 : CH0 >= 32 ? 32 : 16;
    static_assert(CH * BN * 4 <= C::SMEM_BYTES && BM % CH == 0 && CH % 16 == 0, "fp32 row chunk must fit");
    constexpr int NCH = BM / CH, IT = CH * TPR / NTHR;   // chunks per tile, rows-pieces per thread and chunk
    static_assert(IT * NTHR == CH * TPR, "whole row pieces per thread");
    const bf16_t* G13 = static_cast<const bf16_t*>(a.G13);
    bf16_t* dG13 = static_cast<bf16_t*>(a.dG13);
    bf16_t* Ag = static_cast<bf16_t*>(a.Ag);
    float* s_acc = reinterpret_cast<float*>(smem);
    auto off = [&](int row, int q) { return row * BN + ((q ^ (row % NQ4)) << 2); };
    auto unpack = [](uint32_t w, float& lo, float& hi) {
      lo = __uint_as_float(w << 16);
      hi = __uint_as_float(w & 0xFFFF0000u);
    };
    // piece `it` of chunk ch: row (tid + it * NTHR) / TPR of the chunk,
    // columns n0 + 8 * (tid % TPR) ..  The routing indices, then the gates
    // and G13 of all pieces of a chunk are loaded before the chunk is staged.
    // Loads and stores are buffer operations without branches (a piece
    // outside the output reads zeros and stores nowhere through an
    // out-of-range offset), so the compiler can count them and waits only
    // for the data each piece uses.
    const auto r_g13 = make_rsrc(G13, (uint32_t)((size_t)a.M * 2 * I * 2));
    const auto r_dg13 = make_rsrc(dG13, (uint32_t)((size_t)a.M * 2 * I * 2));
    const auto r_ag = make_rsrc(Ag, (uint32_t)((size_t)a.M * I * 2));
    const auto r_part = make_rsrc(a.dgate_part, (uint32_t)((size_t)((I + BN - 1) / BN) * a.M * 4));
    u32x4_t r1[IT], r3[IT];
    float gt[IT];
    int ms[IT];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int c = tid + it * NTHR;
        ms[it] = a.s2f[min(m0 + ch * CH + c / TPR, mlim - 1)];
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int c = tid + it * NTHR;
        const int m = m0 + ch * CH + c / TPR, n = n0 + 8 * (c % TPR);
        const uint32_t o1 = (m < mlim && n < I) ? (uint32_t)(((size_t)m * 2 * I + n) * 2) : OOB;
        gt[it] = a.gate[ms[it]];
        // non-temporal (cache policy 2 = nt): each G13 element is read once
        // (1.5 % faster; the MXFP8 epilogue's fp32 G13 loads measured 3 %
        // slower that way and stay plain)
        r1[it] = __builtin_amdgcn_raw_buffer_load_b128(r_g13, o1, 0, 2);
        r3[it] = __builtin_amdgcn_raw_buffer_load_b128(r_g13, o1 == OOB ? OOB : o1 + I * 2, 0, 2);
      }
      if (ch > 0) __syncthreads();                         // the previous chunk has been read
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if ((wm * WM + 16 * i) / CH != ch) continue;
        const int row = wm * WM + 16 * i + mrow - ch * CH;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          *reinterpret_cast<f32x4_t*>(&s_acc[off(row, (wn * WN + 16 * j + ncol) >> 2)]) = acc[i][j];
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int c = tid + it * NTHR;
        const int row = c / TPR, q = c % TPR;
        const int m = m0 + ch * CH + row, n = n0 + 8 * q;
        const bool ok = m < mlim && n < I;
        const f32x4_t da0 = *reinterpret_cast<const f32x4_t*>(&s_acc[off(row, 2 * q)]);
        const f32x4_t da1 = *reinterpret_cast<const f32x4_t*>(&s_acc[off(row, 2 * q + 1)]);
        const float g = gt[it];
        float g1[8], g3[8], dap[8], d1[8], d3[8], ag[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          unpack(r1[it][w], g1[2 * w], g1[2 * w + 1]);
          unpack(r3[it][w], g3[2 * w], g3[2 * w + 1]);
          dap[w] = da0[w];
          dap[4 + w] = da1[w];
        }
        float part = 0.f;                                  // a piece outside the output reads G13 = 0: adds 0
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float sg = sigmoid_f32(g1[v]);
          const float silu = g1[v] * sg;
          const float av = silu * g3[v];
          part += dap[v] * av;
          const float da = g * dap[v];
          d1[v] = da * g3[v] * sg * (1.f + g1[v] * (1.f - sg));
          d3[v] = da * silu;
          ag[v] = g * av;
        }
        const uint32_t o1 = ok ? (uint32_t)(((size_t)m * 2 * I + n) * 2) : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pack_bf16x2(d1[0], d1[1]), pack_bf16x2(d1[2], d1[3]),
                                                       pack_bf16x2(d1[4], d1[5]), pack_bf16x2(d1[6], d1[7])},
                                               r_dg13, o1, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pack_bf16x2(d3[0], d3[1]), pack_bf16x2(d3[2], d3[3]),
                                                       pack_bf16x2(d3[4], d3[5]), pack_bf16x2(d3[6], d3[7])},
                                               r_dg13, ok ? o1 + I * 2 : OOB, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pack_bf16x2(ag[0], ag[1]), pack_bf16x2(ag[2], ag[3]),
                                                       pack_bf16x2(ag[4], ag[5]), pack_bf16x2(ag[6], ag[7])},
                                               r_ag, ok ? (uint32_t)(((size_t)m * I + n) * 2) : OOB, 0, 0);
        part = fsum_lanes32(part);                         // the 32 lanes of this row
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(part), r_part,
            ((lane & 31) == 0 && m < mlim) ? (uint32_t)(((size_t)(n0 / BN) * a.M + m) * 4) : OOB, 0, 0);
      }
    }
  } else {   // wgrad: fp32 output of one expert, staged through LDS so each
             // store instruction writes whole rows (full cache lines); the
             // tile goes through in chunks of CH rows when it exceeds the LDS
    constexpr int CH0 = C::SMEM_BYTES / (BN * 4);
    constexpr int CH = CH0 >= BM ? BM : CH0 >= 128 ? 128 : CH0 >= 64 ? 64 : CH0 >= 32 ? 32 : 16;
    static_assert(CH * BN * 4 <= C::SMEM_BYTES && BM % CH == 0 && CH % 16 == 0, "fp32 row chunk must fit in the operand LDS");
    float* s_out = reinterpret_cast<float*>(smem);
    constexpr int NQ = BN / 4;                             // 16-byte chunks per row
    auto out_off = [&](int row, int q) { return row * BN + ((q ^ (row % NQ)) << 2); };
    float* out = wout;   // dW[e] or a partial slot of a split expert
    const int ld = (KIND == KIND_WGRAD2) ? I : H;
#pragma unroll
    for (int ch = 0; ch < BM / CH; ++ch) {
      if (ch > 0) __syncthreads();                         // the previous chunk has been read out
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WM + 16 * i + mrow;           // the 16-row block lies in one chunk
        if ((wm * WM + 16 * i) / CH != ch) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int q = (wn * WN + 16 * j + ncol) >> 2;
          *reinterpret_cast<f32x4_t*>(&s_out[out_off(row - ch * CH, q)]) = acc[i][j];
        }
      }
      __syncthreads();
      constexpr int IT = CH * NQ / NTHR;                   // 16-byte pieces per thread and chunk
      static_assert(IT * NTHR == CH * NQ, "whole pieces per thread");
      if (wacc) {   // accumulate-into: every old value of the chunk is loaded before the first store
        f32x4_t old[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int c = tid + it * NTHR, row = c / NQ, q = c % NQ;
          const int m = m0 + ch * CH + row, n = n0 + 4 * q;
          old[it] = (m < mlim && n < nlim) ? *reinterpret_cast<const f32x4_t*>(out + (size_t)m * ld + n)
                                           : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int c = tid + it * NTHR, row = c / NQ, q = c % NQ;
          const int m = m0 + ch * CH + row, n = n0 + 4 * q;
          if (m < mlim && n < nlim)
            st_out<true>(out + (size_t)m * ld + n, old[it] + *reinterpret_cast<const f32x4_t*>(&s_out[out_off(row, q)]));
        }
      } else {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int c = tid + it * NTHR, row = c / NQ, q = c % NQ;
          const int m = m0 + ch * CH + row, n = n0 + 4 * q;
          if (m < mlim && n < nlim)
            st_out<true>(out + (size_t)m * ld + n, *reinterpret_cast<const f32x4_t*>(&s_out[out_off(row, q)]));
        }
      }
    }
  }
}

// Epilogue of the dgrad of W2 in the MXFP8 modes.  The gate-gradient
// partials, the SwiGLU derivative and the gate fold are those of
// gemm_epilogue (from the fp32 G13 these modes save), but instead of dG13 and
// g*A the tile writes their MXFP8 operands of the following GEMMs:
//   dG13 in row blocks of 32 along 2I (A operand of the dgrad of W13): the 4
//     lanes that share a row reduce the block maximum, each lane stores the
//     codes of its 4 consecutive columns;
//   dG13 and g*A in token blocks of 32 (operands of the two weight
//     gradients): the tile's 128 rows are one padded 128-token K tile of the
//     expert (tiles start at the expert's first row, rows past its end count
//     as zeros), the 16 lanes holding a column's block reduce its maximum, the
//     codes are staged transposed in LDS and stored as whole 128-byte rows.
// The values reaching the encoder are those the separate quantisers would
// read, so the codes are the same.
// LDS bytes of the dgrad-of-W2 MXFP8 epilogue's staging (gate-gradient
// partials, transposed code rows and scale bytes of dG13 and g*A)
template <class C>
constexpr int dgrad2_mx8_part_bytes() {   // gate-gradient partials of the WGN column waves
  return C::WGN * C::BM * 4 > 1024 ? C::WGN * C::BM * 4 : 1024;
}
template <class C>
constexpr int dgrad2_mx8_lds_bytes() {
  return dgrad2_mx8_part_bytes<C>() + 3 * C::BN * (C::BM + 16) + 3 * C::BN * (C::BM / 32);
}

template <class C, int LDS>
__device__ __forceinline__ void dgrad2_epilogue_mx8(const LayerArgs& a, const Mx8Args& q,
                                                    f32x4_t (&acc)[C::FM][C::FN], void* smem, int tid, int lane,
                                                    int wm, int wn, int e, int m0, int mlim, int n0) {
  constexpr int BM = C::BM, BN = C::BN, NTHR = C::NTHR, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int NB = BM / 32;                                  // token blocks per tile
  static_assert(BM == MX_KTILE && FM % 2 == 0 && FN % 2 == 0 && WM % 32 == 0, "tile = one padded K tile");
  // staged code rows [column][BM tokens] padded to TS bytes: the 4 column
  // groups of a fragment then fall on different LDS banks
  constexpr int TS = BM + 16;
  constexpr int T_DG = dgrad2_mx8_part_bytes<C>(), T_AG = T_DG + 2 * BN * TS, S_DG = T_AG + BN * TS,
                S_AG = S_DG + 2 * BN * NB;
  static_assert(S_AG + BN * NB == dgrad2_mx8_lds_bytes<C>(), "staging layout");
  static_assert(C::WGN * BM * 4 <= T_DG && S_AG + BN * NB <= LDS, "staging fits in the kernel's LDS");
  uint8_t* lds = static_cast<uint8_t*>(smem);
  const int I = a.I;
  const int mrow = lane & 15, ncol = 4 * (lane >> 4);
  const float* G13 = static_cast<const float*>(a.G13);
  // row codes and scales of dG13 by buffer stores: offsets past the end (OOB)
  // are dropped, which masks rows past the expert and columns past I
  const auto r_qdg = make_rsrc(q.qdg, (uint32_t)a.M * 2 * I);
  const auto r_sdg = make_rsrc(q.sdg, (uint32_t)a.M * 2 * I / 32);
  float psum[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) psum[i] = 0.f;
  // The gates of the wave's rows are loaded up front (the routing index, then
  // the gate), so that each 2x2 block of fragments waits only for its own
  // G13 loads.  Rows past the expert and columns past I read in-bounds
  // values, zeroed below.
  int sfl[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) sfl[i] = a.s2f[min(m0 + wm * WM + 16 * i + mrow, mlim - 1)];
  float gi[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) gi[i] = a.gate[sfl[i]];
  f32x4_t gb[2][2][2];   // [row block ii][column block jj][G1, G3]
  auto load_g13 = [&](int ip, int jp) __attribute__((always_inline)) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int mc = min(m0 + wm * WM + 16 * (2 * ip + ii) + mrow, mlim - 1);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int n = n0 + wn * WN + 16 * (2 * jp + jj) + ncol;
        const size_t o = (size_t)mc * 2 * I + min(n, I - 4);
        gb[ii][jj][0] = *reinterpret_cast<const f32x4_t*>(G13 + o);
        gb[ii][jj][1] = *reinterpret_cast<const f32x4_t*>(G13 + o + I);
      }
    }
  };

#pragma unroll
  for (int ip = 0; ip < FM / 2; ++ip) {
#pragma unroll
    for (int jp = 0; jp < FN / 2; ++jp) {
      load_g13(ip, jp);
      float d[3][2][2][4];   // [dG1, dG3, g*A][row block ii][column block jj][v]; zero outside the expert / I
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * ip + ii;
        const int m = m0 + wm * WM + 16 * i + mrow;
        const float g = gi[i];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int n = n0 + wn * WN + 16 * (2 * jp + jj) + ncol;
          const bool ok = m < mlim && n < I;
          f32x4_t g1 = gb[ii][jj][0];
          f32x4_t g3 = gb[ii][jj][1];
#pragma unroll
          for (int v = 0; v < 4; ++v) {   // zero G13 outside the tile: every derived value is then zero
            g1[v] = ok ? g1[v] : 0.f;
            g3[v] = ok ? g3[v] : 0.f;
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float dap = acc[i][2 * jp + jj][v];
            const float s = sigmoid_f32(g1[v]);
            const float silu = g1[v] * s;
            const float av = silu * g3[v];
            psum[i] += dap * av;
            const float da = g * dap;
            d[0][ii][jj][v] = da * g3[v] * s * (1.f + g1[v] * (1.f - s));
            d[1][ii][jj][v] = da * silu;
            d[2][ii][jj][v] = g * av;
          }
        }
      }
      // row blocks of dG13 (32 columns = fragments 2jp, 2jp+1).  The 4 lanes
      // sharing a row (lane groups g = lane/16) hold codes of the 4 blocks
      // b = 2 ii + h of that row pair: group g has dwords g and 4 + g (columns
      // 4g.., 16 + 4g..) of each.  A 4x4 transpose over the groups (a 32-lane
      // then a 16-lane row swap) gives group g all 8 dwords of block g, stored
      // as two 16-byte pieces with the block's scale byte.
      const int c0 = n0 + wn * WN + 32 * jp;
      uint32_t pk[4][2];   // [block b][jj]: before the transpose, dword g (+4 jj) of block b
      int xs[4];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t amax = 0;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 4; ++v) amax = max(amax, abs_bits(d[h][ii][jj][v]));
          const int X = mx_scale_exp(__uint_as_float(umax_rows4(amax)));
          xs[2 * ii + h] = X;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            pk[2 * ii + h][jj] = mx_pack4(d[h][ii][jj][0], d[h][ii][jj][1], d[h][ii][jj][2], d[h][ii][jj][3], X);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        // groups 2,3 of blocks 0,1 <-> groups 0,1 of blocks 2,3
        auto s = __builtin_amdgcn_permlane32_swap(pk[0][jj], pk[2][jj], false, false);
        pk[0][jj] = s[0];
        pk[2][jj] = s[1];
        s = __builtin_amdgcn_permlane32_swap(pk[1][jj], pk[3][jj], false, false);
        pk[1][jj] = s[0];
        pk[3][jj] = s[1];
        // groups 1,3 of blocks 0,2 <-> groups 0,2 of blocks 1,3
        s = __builtin_amdgcn_permlane16_swap(pk[0][jj], pk[1][jj], false, false);
        pk[0][jj] = s[0];
        pk[1][jj] = s[1];
        s = __builtin_amdgcn_permlane16_swap(pk[2][jj], pk[3][jj], false, false);
        pk[2][jj] = s[0];
        pk[3][jj] = s[1];
      }
      {   // now pk[r][jj] of group g = dword r (+4 jj) of block g
        const int g = lane >> 4;
        const int m = m0 + wm * WM + 16 * (2 * ip + (g >> 1)) + mrow;
        const bool ok = m < mlim && c0 < I;
        const uint32_t row = (uint32_t)m * 2 * I + (g & 1) * I + c0;
        const int X = g == 0 ? xs[0] : g == 1 ? xs[1] : g == 2 ? xs[2] : xs[3];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pk[0][jj], pk[1][jj], pk[2][jj], pk[3][jj]}, r_qdg,
                                                 ok ? row + 16 * jj : OOB, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(X + 127), r_sdg, ok ? row / 32 : OOB, 0, 0);
      }
      // token blocks (32 rows = fragments 2ip, 2ip+1; 16 lanes per column), staged in LDS.
      // The 24 maxima of this sub-block advance through the DPP steps together.
      const int tl = wm * WM + 32 * ip + mrow;                 // tile token of row block 0
      uint32_t am[2][3][4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int h = 0; h < 3; ++h)
#pragma unroll
          for (int v = 0; v < 4; ++v) am[jj][h][v] = max(abs_bits(d[h][0][jj][v]), abs_bits(d[h][1][jj][v]));
      row16_umax_steps(am);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
        for (int h = 0; h < 3; ++h) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int X = mx_scale_exp(__uint_as_float(am[jj][h][v]));
            const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(d[h][0][jj][v], -X),
                                                                         ldexpf(d[h][1][jj][v], -X), 0, false);
            const int cl = wn * WN + 16 * (2 * jp + jj) + ncol + v;   // tile column
            uint8_t* t = lds + (h == 2 ? T_AG + cl * TS : T_DG + (h * BN + cl) * TS);
            t[tl] = (uint8_t)(w & 0xFFu);
            t[tl + 16] = (uint8_t)((w >> 8) & 0xFFu);
            if (mrow == 0)
              lds[(h == 2 ? S_AG + cl * NB : S_DG + (h * BN + cl) * NB) + wm * (WM / 32) + ip] = (uint8_t)(X + 127);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one 2x2 block of fragments live at a time
    }
  }

  dgate_partials<C>(a, psum, reinterpret_cast<float*>(lds), tid, lane, wm, wn, m0, mlim, n0);   // ends with a barrier

  // the staged token blocks -> the transposed operands, whole rows of the K tile
  const size_t Mp = (size_t)q.Mp;
  const size_t p0 = (size_t)q.pad_off[e] + (size_t)(m0 - a.offsets[e]);
  uint8_t* qdgt = const_cast<uint8_t*>(q.qdgt);
  uint8_t* sdgt = const_cast<uint8_t*>(q.sdgt);
  uint8_t* qagt = const_cast<uint8_t*>(q.qagt);
  uint8_t* sagt = const_cast<uint8_t*>(q.sagt);
  for (int idx = tid; idx < 3 * BN * (BM / 16); idx += NTHR) {
    const int col = idx / (BM / 16), ch = idx % (BM / 16);   // col < 2 BN: dG1 | dG3, then g*A
    const int c = n0 + col % BN;
    if (c >= I) continue;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + (col < 2 * BN ? T_DG + col * TS : T_AG + (col - 2 * BN) * TS) + 16 * ch);
    uint8_t* dst = col < 2 * BN ? qdgt + (size_t)(col < BN ? c : I + c) * Mp : qagt + (size_t)c * Mp;
    *reinterpret_cast<u32x4_t*>(dst + p0 + 16 * ch) = v;
  }
  for (int col = tid; col < 3 * BN; col += NTHR) {
    const int c = n0 + col % BN;
    if (c >= I) continue;
    const uint32_t v = *reinterpret_cast<const uint32_t*>(lds + (col < 2 * BN ? S_DG + col * NB : S_AG + (col - 2 * BN) * NB));
    uint8_t* dst = col < 2 * BN ? sdgt + (size_t)(col < BN ? c : I + c) * (Mp / 32) : sagt + (size_t)c * (Mp / 32);
    *reinterpret_cast<uint32_t*>(dst + p0 / 32) = v;
  }
}

}  // namespace gg
}  // namespace moe
