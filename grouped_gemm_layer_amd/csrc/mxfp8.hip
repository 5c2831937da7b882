// MXFP8 quantisation of the backward GEMM operands (fp8_bwd mode).
//
// Group-aware MXFP8 quantisation (TE dropless-MoE page, "03 Specialised
// optimisations": group-aware MXFP8 quantisation feeding MXFP8 grouped GEMM):
// every operand is cut into blocks of 32 consecutive elements along its GEMM's
// K; a block stores one E8M0 scale 2^X and 32 E4M3FN codes.
//   X    = smallest integer with amax <= 448 * 2^X (clamped to [-127, 127];
//          an all-zero block gets X = -127)
//   code = v / 2^X rounded to the nearest E4M3FN value (ties to even),
//          saturating at 448; the sign bit is kept also for values rounding to 0.
// Blocks along the token dimension start at each expert's first row; the
// expert's last block is zero-padded ("group-aware"), and so is the gap up to
// the next multiple of MX_KTILE where the next expert starts.
//
// Layouts written here (bytes): codes [rows][K], scales [rows][K/32], K the
// operand's GEMM-K (contiguous).  The scaling by 2^-X is exact (ldexp) and the
// E4M3 rounding is the hardware conversion (nearest, ties to even), so the
// codes are those of the exact definition for the same inputs.
#include "mx_codec.h"

namespace moe {

__device__ __forceinline__ void unpack_bf16x8(const uint4 r, float* out) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// 16-byte source load; NT = non-temporal, for sources read once (the
// weights: W13 0.30 -> 0.28 ms, W2 0.15 -> 0.13 for both layouts).  The
// gathered token rows, read once per routed slot, stay cached (non-temporal
// there: 0.13 -> 0.17 ms).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
template <bool NT = false>
__device__ __forceinline__ uint4 ld16(const void* p) {
  u32x4v w;
  if constexpr (NT) w = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  else w = *reinterpret_cast<const u32x4v*>(p);
  return make_uint4(w.x, w.y, w.z, w.w);
}

// 32 consecutive elements of a row, bf16 or fp32
__device__ __forceinline__ void load32(const bf16_t* p, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack_bf16x8(ld16(p + 8 * i), v + 8 * i);
}
__device__ __forceinline__ void load32(const float* p, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 w = ld16(p + 4 * i);
    v[4 * i] = __uint_as_float(w.x); v[4 * i + 1] = __uint_as_float(w.y);
    v[4 * i + 2] = __uint_as_float(w.z); v[4 * i + 3] = __uint_as_float(w.w);
  }
}

// Row-wise: block = 32 consecutive elements of a row.  Source row r is
// src_row(r) = s2f[r] / k when s2f is given (gathered dY rows), else r.
template <typename T>
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const T* __restrict__ src, int R, int K,
                                                            const int32_t* __restrict__ s2f, int k,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int nb = K / 32;
  const long total = (long)R * nb;
  for (long t = (long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long)gridDim.x * 256) {
    const int r = (int)(t / nb), b = (int)(t % nb);
    const int sr = s2f ? s2f[r] / k : r;
    float v[32];
    load32(src + (size_t)sr * K + 32 * b, v);
    uint32_t packed[8];
    const uint32_t s = mx_quant_block(v, packed);
    uint4* o = reinterpret_cast<uint4*>(codes + (size_t)r * K + 32 * b);
    o[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    o[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    scales[(size_t)r * nb + b] = (uint8_t)s;
  }
}

// Padded token offsets: pad_off[e] = sum_{e' < e} ceil(count_e' / MX_KTILE) * MX_KTILE.
__global__ __launch_bounds__(512) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                          int32_t* __restrict__ pad_off) {
  __shared__ int s[2][513];
  const int e = threadIdx.x;
  int cur = 0;
  s[0][e] = (e < E) ? (offsets[e + 1] - offsets[e] + MX_KTILE - 1) / MX_KTILE * MX_KTILE : 0;
  if (e == 0) s[0][512] = 0;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    int val = s[cur][e];
    if (e >= off) val += s[cur][e - off];
    s[cur ^ 1][e] = val;
    cur ^= 1;
    __syncthreads();
  }
  if (e < E) pad_off[e + 1] = s[cur][e];
  if (e == 0) pad_off[0] = 0;
}

// Transposing quantiser: blocks of 32 run down the rows of the source and
// the output is written transposed (feature-major), K = the source's rows.
//   GROUPED: source rows r of the expert-sorted order (read as
//     src[s2f[r] / k] when s2f is given: gathered x / dY rows); expert e's
//     rows go to output columns pad_off[e] .., the gap up to pad_off[e+1]
//     holds zero codes; n_ptiles = padded tiles of MX_KTILE columns.
//   dense: tile expert e (n_e of them) of a [E][Kd][F] source, rows e*Kd + p;
//     output [E][F][Kd]; n_ptiles = Kd / MX_KTILE.
// A tile of MX_KTILE rows x QT_F features is staged in LDS as fp32 with
// coalesced 16-byte row loads; thread (f, q) then quantises feature f over
// the 32 rows of block q, and the codes and scales leave through LDS along
// the output rows.
constexpr int QT_F = 64;            // features per tile
// LDS row stride of the source tile (elements of the source type, which the
// tile keeps: bf16 is staged as is): rows stay 16-byte aligned
template <typename T> constexpr int qt_ld() { return QT_F + 16 / (int)sizeof(T); }
constexpr int QT_CLD = MX_KTILE + 16;   // LDS row stride of the staged codes (bytes)
constexpr int QT_RLD = QT_F + 16;       // LDS row stride of the staged row-wise codes (bytes)

template <typename T, bool GROUPED, bool ROWS = false>
__global__ __launch_bounds__(256) void mx_quant_t_kernel(const T* __restrict__ src, int F,
                                                         const int32_t* __restrict__ s2f, int k,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ pad_off, int E, int Kd,
                                                         int ld_out, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         int n_ptiles, int n_e,
                                                         uint8_t* __restrict__ row_codes = nullptr,
                                                         uint8_t* __restrict__ row_scales = nullptr) {
  constexpr int QT_LD = qt_ld<T>();
  __shared__ __attribute__((aligned(16))) T s_tile[MX_KTILE * QT_LD];
  __shared__ int s_src[MX_KTILE];       // source row of each tile row, -1 = padding
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[QT_F * QT_CLD];   // codes [feature][tile row]
  __shared__ __attribute__((aligned(4))) uint8_t s_scales[QT_F * 4];        // scales [feature][block]
  // row-wise codes / scales of the tile (ROWS only)
  __shared__ __attribute__((aligned(16))) uint8_t s_rcodes[ROWS ? MX_KTILE * QT_RLD : 16];
  __shared__ __attribute__((aligned(4))) uint8_t s_rscales[ROWS ? MX_KTILE * 2 : 4];
  // 1-D grid of nf x np x ne tiles (features fastest).  Dense sources are
  // renumbered so that each XCD (blocks are dealt round-robin to the 8 XCDs)
  // takes a contiguous run of tiles: neighbouring feature tiles, whose
  // row-wise output shares lines, then meet in one L2 (measured faster; the
  // gathered token tiles run faster in launch order)
  const int per_xcd = gridDim.x / 8;
  const int L = GROUPED ? (int)blockIdx.x : (int)(blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
  const int nf = (F + QT_F - 1) / QT_F;
  if (L >= nf * n_ptiles * n_e) return;
  const int tf = L % nf, tp = (L / nf) % n_ptiles, te = L / (nf * n_ptiles);
  const int f0 = tf * QT_F;
  const int p0 = MX_KTILE * tp;
  size_t out_base = 0, sc_base = 0;
  if constexpr (GROUPED) {
    if (p0 >= pad_off[E]) return;       // uniform over the block
    int lo = 0, hi = E - 1;             // expert e with pad_off[e] <= p0 < pad_off[e+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pad_off[mid] <= p0) lo = mid; else hi = mid - 1;
    }
    if (threadIdx.x < MX_KTILE) {
      const int r = offsets[lo] + (p0 - pad_off[lo]) + threadIdx.x;
      s_src[threadIdx.x] = (r < offsets[lo + 1]) ? (s2f ? s2f[r] / k : r) : -1;
    }
  } else {
    const int e = te;
    if (threadIdx.x < MX_KTILE) s_src[threadIdx.x] = e * Kd + p0 + threadIdx.x;
    out_base = (size_t)e * F * ld_out;
    sc_base = (size_t)e * F * (ld_out / 32);
  }
  __syncthreads();

  // rows -> LDS: every load of the thread is issued before the first store
  constexpr int EPC = 16 / (int)sizeof(T);      // values per 16-byte chunk
  constexpr int CPR = QT_F / EPC;               // chunks per tile row
  constexpr int RPP = 256 / CPR;                // tile rows per pass
  constexpr int NP = MX_KTILE / RPP;            // passes
  const int c = threadIdx.x % CPR, fc = f0 + c * EPC, r0 = threadIdx.x / CPR;
  if ((F % EPC) == 0) {                         // rows 16-byte aligned, chunks never straddle F
    uint4 raw[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int sr = s_src[r0 + p * RPP];
      raw[p] = (sr >= 0 && fc < F) ? ld16<!GROUPED>(src + (size_t)sr * F + fc) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<uint4*>(&s_tile[(r0 + p * RPP) * QT_LD + c * EPC]) = raw[p];
  } else {
    for (int r = r0; r < MX_KTILE; r += RPP) {
      const int sr = s_src[r];
#pragma unroll
      for (int i = 0; i < EPC; ++i)
        s_tile[r * QT_LD + c * EPC + i] = (sr >= 0 && fc + i < F) ? src[(size_t)sr * F + fc + i] : T(0);
    }
  }
  __syncthreads();

  if constexpr (ROWS) {
    // the same tile quantised along its rows as well (dense sources, F a
    // multiple of QT_F): thread = one tile row x one block of 32 features
    static_assert(!GROUPED && 2 * MX_KTILE == 256, "two row blocks per tile row");
    const int r = threadIdx.x % MX_KTILE, b = threadIdx.x / MX_KTILE;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; i += EPC) {
      const uint4 t = *reinterpret_cast<const uint4*>(&s_tile[r * QT_LD + 32 * b + i]);
      if constexpr (sizeof(T) == 2) {
        unpack_bf16x8(t, v + i);
      } else {
        v[i] = __uint_as_float(t.x); v[i + 1] = __uint_as_float(t.y);
        v[i + 2] = __uint_as_float(t.z); v[i + 3] = __uint_as_float(t.w);
      }
    }
    uint32_t packed[8];
    const uint32_t sc = mx_quant_block(v, packed);
    // staged in LDS, then stored along the rows: 4 lanes per 64-byte row piece
    uint4* d = reinterpret_cast<uint4*>(&s_rcodes[r * QT_RLD + 32 * b]);
    d[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    d[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    s_rscales[2 * r + b] = (uint8_t)sc;
    __syncthreads();
    const size_t row0 = (size_t)te * Kd + p0;
#pragma unroll
    for (int i = threadIdx.x; i < MX_KTILE * (QT_F / 16); i += 256) {
      const int rr = i / (QT_F / 16), ch = i % (QT_F / 16);
      *reinterpret_cast<uint4*>(row_codes + (row0 + rr) * F + f0 + 16 * ch) =
          *reinterpret_cast<const uint4*>(&s_rcodes[rr * QT_RLD + 16 * ch]);
    }
    if (threadIdx.x < MX_KTILE)
      *reinterpret_cast<uint16_t*>(row_scales + (row0 + threadIdx.x) * (F / 32) + f0 / 32) =
          *reinterpret_cast<const uint16_t*>(&s_rscales[2 * threadIdx.x]);
  }

  // one feature x one block of 32 rows per thread (a wave = 64 features of one
  // block); codes and scales are staged in LDS so that the stores run along
  // the output rows (8 lanes per 128-byte row of the tile)
  const int f = threadIdx.x % QT_F, q = threadIdx.x / QT_F;
  {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = ElemTraits<T>::load(&s_tile[(32 * q + i) * QT_LD + f]);
    uint32_t packed[8];
    const uint32_t sc = mx_quant_block(v, packed);
    uint4* d = reinterpret_cast<uint4*>(&s_codes[f * QT_CLD + 32 * q]);
    d[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    d[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    s_scales[f * 4 + q] = (uint8_t)sc;
  }
  __syncthreads();
  constexpr int CPT = MX_KTILE / 16;             // 16-byte chunks per output row of the tile
#pragma unroll
  for (int i = threadIdx.x; i < QT_F * CPT; i += 256) {
    const int ff = i / CPT, ch = i % CPT;
    if (f0 + ff < F)
      *reinterpret_cast<uint4*>(codes + out_base + (size_t)(f0 + ff) * ld_out + p0 + 16 * ch) =
          *reinterpret_cast<const uint4*>(&s_codes[ff * QT_CLD + 16 * ch]);
  }
  if (threadIdx.x < QT_F && f0 + threadIdx.x < F)
    *reinterpret_cast<uint32_t*>(scales + sc_base + (size_t)(f0 + threadIdx.x) * (ld_out / 32) + p0 / 32) =
        *reinterpret_cast<const uint32_t*>(&s_scales[threadIdx.x * 4]);
}

template <typename T>
hipError_t launch_mx_quant_rows(const T* src, int R, int K, const int32_t* s2f, int k, uint8_t* codes,
                                uint8_t* scales, hipStream_t s) {
  const long total = (long)R * (K / 32);
  const int grid = (int)min((total + 255) / 256, (long)65536);
  return launch_kernel(mx_quant_rows_kernel<T>, dim3(grid), dim3(256), 0, s, src, R, K, s2f, k, codes, scales);
}
template hipError_t launch_mx_quant_rows<bf16_t>(const bf16_t*, int, int, const int32_t*, int, uint8_t*, uint8_t*,
                                                 hipStream_t);

// blocks for nf x np x ne tiles, a multiple of the 8 XCDs
inline int qt_grid(int F, int np, int ne) {
  const long tiles = (long)((F + QT_F - 1) / QT_F) * np * ne;
  return (int)((tiles + 7) / 8 * 8);
}

hipError_t launch_mx_quant_cols_t(const bf16_t* src, int E, int Kd, int N, uint8_t* codes, uint8_t* scales,
                                  hipStream_t s) {
  return launch_kernel((mx_quant_t_kernel<bf16_t, false>), dim3(qt_grid(N, Kd / MX_KTILE, E)), dim3(256), 0, s, src,
                     N, nullptr, 1, nullptr, nullptr, E, Kd, Kd, codes, scales, Kd / MX_KTILE, E, nullptr, nullptr);
}

hipError_t launch_mx_quant_both(const bf16_t* src, int E, int Kd, int N, uint8_t* codes_t, uint8_t* scales_t,
                                uint8_t* codes_r, uint8_t* scales_r, hipStream_t s) {
  return launch_kernel((mx_quant_t_kernel<bf16_t, false, true>), dim3(qt_grid(N, Kd / MX_KTILE, E)), dim3(256), 0, s,
                     src, N, nullptr, 1, nullptr, nullptr, E, Kd, Kd, codes_t, scales_t, Kd / MX_KTILE, E, codes_r,
                     scales_r);
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* pad_off, hipStream_t s) {
  return launch_kernel(pad_offsets_kernel, dim3(1), dim3(512), 0, s, offsets, E, pad_off);
}

template <typename T>
hipError_t launch_mx_quant_tokens_t(const T* src, int F, const int32_t* s2f, int k, const int32_t* offsets,
                                    const int32_t* pad_off, int E, int Mp, uint8_t* codes, uint8_t* scales,
                                    hipStream_t s) {
  return launch_kernel((mx_quant_t_kernel<T, true>), dim3(qt_grid(F, Mp / MX_KTILE, 1)), dim3(256), 0, s, src, F, s2f,
                     k, offsets, pad_off, E, 0, Mp, codes, scales, Mp / MX_KTILE, 1, nullptr, nullptr);
}
template hipError_t launch_mx_quant_tokens_t<bf16_t>(const bf16_t*, int, const int32_t*, int, const int32_t*,
                                                     const int32_t*, int, int, uint8_t*, uint8_t*, hipStream_t);

}  // namespace moe
