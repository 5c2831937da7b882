// Ragged grouped GEMMs of the MoE layer on bf16 MFMA (gfx950,
// v_mfma_f32_16x16x32_bf16), fp32 accumulation, with the layer's epilogues
// fused: SwiGLU after the W1/W3 GEMM; gate-gradient partials, gate folding
// and the SwiGLU derivative after the dgrad GEMM of W2.
//
// The grouped GEMM runs all experts in one launch over the actual per-expert
// row counts read on the device (TE dropless-MoE page, "Optimisation 1:
// Grouped GEMM"); SwiGLU is fused between the two expert linear layers (Prime
// Mega MoE news page, "How does the fused kernel work?").  The token gather of
// the dispatch is fused into the operand loads (rows are read from x or dY
// through the routing map), so the permuted copies are never written.
//
// Every kernel computes C[m][n] = sum_k A[m][k] B[n][k] over one 128x128 tile:
//   row-ragged kinds (forward, dgrad): m = expert-sorted token rows of one
//     expert (tile table), n = output features, K = H, I or 2I;
//   wgrad kinds: m, n = weight-gradient rows/cols of one expert (grid.y),
//     K = that expert's token rows, ragged and zero-padded.
// Operands come in two global layouts:
//   KC: element (row, k) at row_ptr(row)[k]        (K contiguous)
//   KO: element (row, k) at krow_ptr(k)[row]       (rows contiguous, "transposed")
// Both are staged to LDS as [row][k] (64 k per row, 16-byte chunks XOR
// swizzled by row) so every MFMA operand is one 16-byte LDS read; KO tiles are
// transposed in registers (4 k x 8 rows per thread) on the way in.
//
// Four waves as 2x2, each owning a 64x64 sub-tile = 4x4 MFMA blocks of 16x16.
// The MFMA's first operand is the B tile (rows n) and its second the A tile
// (rows m), so lane l holds D[n = 4*(l/16) + v][m = l%16]: four consecutive
// output features of one row, stored as one 8- or 16-byte write.
// Main loop: global loads of tile k+1 into registers overlap the MFMAs of
// tile k; one barrier per K step (double-buffered LDS).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = BF16_BM;   // 128
constexpr int BN = BF16_BN;   // 128
constexpr int BK = 64;
constexpr int NTHR = 256;
constexpr int WM = BM / 2, WN = BN / 2;
constexpr int FM = WM / 16, FN = WN / 16;
static_assert(BM == 128 && BN == 128, "loaders assume 128-row tiles");

// element offset of (row, 8-element chunk) inside a [rows][BK] LDS tile
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 3);
}

template <int KIND> struct KindTraits;
// A = gathered x rows (KC), B = W13 rows (KC, G1/G3 paired), K = H
template <> struct KindTraits<KIND_FWD1> { static constexpr bool ragged_rows = true, a_ko = false, b_ko = false; };
// A = A rows (KC), B = W2 rows (KC), K = I
template <> struct KindTraits<KIND_FWD2> { static constexpr bool ragged_rows = true, a_ko = false, b_ko = false; };
// A = gathered dY rows (KC), B[n=i][k=h] = W2[h][i] (KO), K = H
template <> struct KindTraits<KIND_DGRAD2> { static constexpr bool ragged_rows = true, a_ko = false, b_ko = true; };
// A = dG13 rows (KC), B[n=h][k=j] = W13[j][h] (KO), K = 2I
template <> struct KindTraits<KIND_DGRAD1> { static constexpr bool ragged_rows = true, a_ko = false, b_ko = true; };
// A[m=h][k=r] = dY[t(r)][h] (KO), B[n=i][k=r] = Ag[r][i] (KO)
template <> struct KindTraits<KIND_WGRAD2> { static constexpr bool ragged_rows = false, a_ko = true, b_ko = true; };
// A[m=j][k=r] = dG13[r][j] (KO), B[n=h][k=r] = x[t(r)][h] (KO)
template <> struct KindTraits<KIND_WGRAD1> { static constexpr bool ragged_rows = false, a_ko = true, b_ko = true; };

// KC loader: 128 rows x 64 k; thread handles rows (tid>>3) + 32*i, chunk tid&7.
struct KcLoader {
  const bf16_t* p[4];   // row base (already offset by chunk), nullptr = zero row
  uint4 r[4];
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (p[i]) r[i] = *reinterpret_cast<const uint4*>(p[i] + kt * BK);
      else r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(lds + lds_off(row, tid & 7)) = r[i];
    }
  }
};

// KO loader: 64 k x 128 rows; thread handles k = 4q..4q+3 (q = tid>>4) and
// rows 8c..8c+7 (c = tid&15).  Transposed to [row][k] on the LDS store.
struct KoLoader {
  uint4 r[4];
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    const int q = tid >> 4, c = tid & 15;
    const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
    const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
    const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      uint32_t lo, hi;
      if (j & 1) {
        lo = (w0[d] >> 16) | (w1[d] & 0xFFFF0000u);
        hi = (w2[d] >> 16) | (w3[d] & 0xFFFF0000u);
      } else {
        lo = (w0[d] & 0xFFFFu) | (w1[d] << 16);
        hi = (w2[d] & 0xFFFFu) | (w3[d] << 16);
      }
      const int row = 8 * c + j;
      *reinterpret_cast<uint2*>(lds + lds_off(row, q >> 1) + 4 * (q & 1)) = make_uint2(lo, hi);
    }
  }
};

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

template <int KIND>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(LayerArgs a, int n_tiles) {
  using Tr = KindTraits<KIND>;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];
  // after the main loop's last barrier the A tiles are free: reused for the
  // gate-gradient reduction of the dgrad epilogue
  float* s_part = reinterpret_cast<float*>(&sA[0][0]);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int H = a.H, I = a.I, k = a.k;

  // ---------------- tile decode ----------------
  int e, m0, mlim, n0, klo = 0, khi = 0, nk;
  if constexpr (Tr::ragged_rows) {
    const int nt = blockIdx.x % n_tiles;
    const int mt = blockIdx.x / n_tiles;
    e = a.tile_expert[mt];
    if (e < 0) return;
    m0 = a.tile_row0[mt];
    mlim = a.offsets[e + 1];
    n0 = nt * (KIND == KIND_FWD1 ? BN / 2 : BN);
    const int K = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2) ? H : (KIND == KIND_FWD2 ? I : 2 * I);
    nk = K / BK;
  } else {
    e = blockIdx.y;
    const int nt = blockIdx.x % n_tiles;
    const int mt = blockIdx.x / n_tiles;
    m0 = mt * BM;
    n0 = nt * BN;
    klo = a.offsets[e];
    khi = a.offsets[e + 1];
    nk = (khi - klo + BK - 1) / BK;
    mlim = (KIND == KIND_WGRAD2) ? H : 2 * I;
  }
  // valid extent along n
  const int nlim = (KIND == KIND_FWD1) ? I
                 : (KIND == KIND_FWD2 || KIND == KIND_DGRAD1) ? H
                 : (KIND == KIND_DGRAD2) ? I
                 : (KIND == KIND_WGRAD2) ? I : H;

  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* dy = static_cast<const bf16_t*>(a.dy);
  const bf16_t* w13 = static_cast<const bf16_t*>(a.w13) + (size_t)e * 2 * I * H;
  const bf16_t* w2 = static_cast<const bf16_t*>(a.w2) + (size_t)e * H * I;

  // ---------------- operand setup ----------------
  KcLoader la{}, lb{};
  KoLoader oa{}, ob{};
  if constexpr (!Tr::a_ko) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + (tid >> 3) + 32 * i;
      const bf16_t* p = nullptr;
      if (row < mlim) {
        if constexpr (KIND == KIND_FWD1) p = x + (size_t)(a.s2f[row] / k) * H;
        else if constexpr (KIND == KIND_DGRAD2) p = dy + (size_t)(a.s2f[row] / k) * H;
        else if constexpr (KIND == KIND_FWD2) p = static_cast<const bf16_t*>(a.A) + (size_t)row * I;
        else p = static_cast<const bf16_t*>(a.dG13) + (size_t)row * 2 * I;
        p += (tid & 7) * 8;
      }
      la.p[i] = p;
    }
  }
  if constexpr (!Tr::b_ko) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = (tid >> 3) + 32 * i;
      const bf16_t* p = nullptr;
      if constexpr (KIND == KIND_FWD1) {
        const int c = n0 + (nn & (BN / 2 - 1));
        if (c < I) p = w13 + (size_t)((nn < BN / 2) ? c : I + c) * H;
      } else {  // FWD2
        const int n = n0 + nn;
        if (n < H) p = w2 + (size_t)n * I;
      }
      if (p) p += (tid & 7) * 8;
      lb.p[i] = p;
    }
  }
  // KO loads: k rows kbase + 4q + i, columns col0 + 8c
  const int q = tid >> 4, c8 = (tid & 15) * 8;
  auto load_ko_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = klo + kt * BK + 4 * q + i;
      const int col = m0 + c8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < khi && col < mlim) {
        const bf16_t* p;
        if constexpr (KIND == KIND_WGRAD2) p = dy + (size_t)(a.s2f[r] / k) * H + col;
        else p = static_cast<const bf16_t*>(a.dG13) + (size_t)r * 2 * I + col;
        v = *reinterpret_cast<const uint4*>(p);
      }
      oa.r[i] = v;
    }
  };
  auto load_ko_b = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = n0 + c8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if constexpr (Tr::ragged_rows) {   // dense K of the weights
        const int kr = kt * BK + 4 * q + i;
        if (col < nlim) {
          const bf16_t* p;
          if constexpr (KIND == KIND_DGRAD2) p = w2 + (size_t)kr * I + col;
          else p = w13 + (size_t)kr * H + col;
          v = *reinterpret_cast<const uint4*>(p);
        }
      } else {
        const int r = klo + kt * BK + 4 * q + i;
        if (r < khi && col < nlim) {
          const bf16_t* p;
          if constexpr (KIND == KIND_WGRAD2) p = static_cast<const bf16_t*>(a.Ag) + (size_t)r * I + col;
          else p = x + (size_t)(a.s2f[r] / k) * H + col;
          v = *reinterpret_cast<const uint4*>(p);
        }
      }
      ob.r[i] = v;
    }
  };
  auto load_tile = [&](int kt) {
    if constexpr (Tr::a_ko) load_ko_a(kt); else la.load(kt);
    if constexpr (Tr::b_ko) load_ko_b(kt); else lb.load(kt);
  };
  auto store_tile = [&](int buf) {
    if constexpr (Tr::a_ko) oa.store(sA[buf], tid); else la.store(sA[buf], tid);
    if constexpr (Tr::b_ko) ob.store(sB[buf], tid); else lb.store(sB[buf], tid);
  };

  // LDS row of the j-th 16-row MFMA block of this wave's B sub-tile
  auto brow = [&](int j) -> int {
    if constexpr (KIND == KIND_FWD1) {
      return (j < FN / 2) ? wn * (WN / 2) + 16 * j : BN / 2 + wn * (WN / 2) + 16 * (j - FN / 2);
    } else {
      return wn * WN + 16 * j;
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const bf16_t* As = sA[buf];
    const bf16_t* Bs = sB[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int chunk = ks * 4 + (lane >> 4);
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm * WM + 16 * i + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(brow(j) + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---------------- epilogues ----------------
  const int mrow = lane & 15;         // row inside a 16x16 block
  const int ncol = 4 * (lane >> 4);   // first of 4 consecutive columns

  if constexpr (KIND == KIND_FWD1) {
    bf16_t* G13 = static_cast<bf16_t*>(a.G13);
    bf16_t* Aout = static_cast<bf16_t*>(a.A);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * WM + 16 * i + mrow;
      if (m >= mlim) continue;
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int c = n0 + wn * (WN / 2) + 16 * j + ncol;
        if (c >= I) continue;
        const f32x4_t g1 = acc[i][j], g3 = acc[i][j + FN / 2];
        float av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) av[v] = g1[v] * sigmoid_f32(g1[v]) * g3[v];
        *reinterpret_cast<uint2*>(G13 + (size_t)m * 2 * I + c) = pack4(g1[0], g1[1], g1[2], g1[3]);
        *reinterpret_cast<uint2*>(G13 + (size_t)m * 2 * I + I + c) = pack4(g3[0], g3[1], g3[2], g3[3]);
        *reinterpret_cast<uint2*>(Aout + (size_t)m * I + c) = pack4(av[0], av[1], av[2], av[3]);
      }
    }
  } else if constexpr (KIND == KIND_FWD2 || KIND == KIND_DGRAD1) {
    bf16_t* out = static_cast<bf16_t*>(KIND == KIND_FWD2 ? a.O : a.dXp);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * WM + 16 * i + mrow;
      if (m >= mlim) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WN + 16 * j + ncol;
        if (n >= nlim) continue;
        const f32x4_t v = acc[i][j];
        *reinterpret_cast<uint2*>(out + (size_t)m * H + n) = pack4(v[0], v[1], v[2], v[3]);
      }
    }
  } else if constexpr (KIND == KIND_DGRAD2) {
    const bf16_t* G13 = static_cast<const bf16_t*>(a.G13);
    bf16_t* dG13 = static_cast<bf16_t*>(a.dG13);
    bf16_t* Ag = static_cast<bf16_t*>(a.Ag);
    float psum[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      psum[i] = 0.f;
      const int m = m0 + wm * WM + 16 * i + mrow;
      if (m >= mlim) continue;
      const float g = a.gate[a.s2f[m]];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WN + 16 * j + ncol;
        if (n >= I) continue;
        const uint2 r1 = *reinterpret_cast<const uint2*>(G13 + (size_t)m * 2 * I + n);
        const uint2 r3 = *reinterpret_cast<const uint2*>(G13 + (size_t)m * 2 * I + I + n);
        const float g1v[4] = {__uint_as_float(r1.x << 16), __uint_as_float(r1.x & 0xFFFF0000u),
                              __uint_as_float(r1.y << 16), __uint_as_float(r1.y & 0xFFFF0000u)};
        const float g3v[4] = {__uint_as_float(r3.x << 16), __uint_as_float(r3.x & 0xFFFF0000u),
                              __uint_as_float(r3.y << 16), __uint_as_float(r3.y & 0xFFFF0000u)};
        float d1[4], d3[4], ag[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float dap = acc[i][j][v];
          const float s = sigmoid_f32(g1v[v]);
          const float silu = g1v[v] * s;
          const float av = silu * g3v[v];
          psum[i] += dap * av;
          const float da = g * dap;
          d1[v] = da * g3v[v] * s * (1.f + g1v[v] * (1.f - s));
          d3[v] = da * silu;
          ag[v] = g * av;
        }
        *reinterpret_cast<uint2*>(dG13 + (size_t)m * 2 * I + n) = pack4(d1[0], d1[1], d1[2], d1[3]);
        *reinterpret_cast<uint2*>(dG13 + (size_t)m * 2 * I + I + n) = pack4(d3[0], d3[1], d3[2], d3[3]);
        *reinterpret_cast<uint2*>(Ag + (size_t)m * I + n) = pack4(ag[0], ag[1], ag[2], ag[3]);
      }
    }
    // reduce the gate-gradient partial over this tile's n: lanes sharing a row,
    // then the two waves of a row block (fixed order: deterministic)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      psum[i] += __shfl_xor(psum[i], 16);
      psum[i] += __shfl_xor(psum[i], 32);
    }
    if (wn == 1 && lane < 16) {
#pragma unroll
      for (int i = 0; i < FM; ++i) s_part[wm * WM + 16 * i + lane] = psum[i];
    }
    __syncthreads();
    if (wn == 0 && lane < 16) {
      const int nt = n0 / BN;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int ml = wm * WM + 16 * i + lane;
        const int m = m0 + ml;
        if (m < mlim) a.dgate_part[(size_t)nt * a.M + m] = psum[i] + s_part[ml];
      }
    }
  } else {   // wgrad: fp32 output of one expert
    float* out = (KIND == KIND_WGRAD2) ? a.dw2 + (size_t)e * H * I : a.dw13 + (size_t)e * 2 * I * H;
    const int ld = (KIND == KIND_WGRAD2) ? I : H;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * WM + 16 * i + mrow;
      if (m >= mlim) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WN + 16 * j + ncol;
        if (n >= nlim) continue;
        const f32x4_t v = acc[i][j];
        *reinterpret_cast<float4*>(out + (size_t)m * ld + n) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(GemmKind kind, const LayerArgs& a, hipStream_t s) {
  const int max_mt = max_row_tiles(a.M, a.E, BM);
  switch (kind) {
    case KIND_FWD1: {
      const int nt = (a.I + BN / 2 - 1) / (BN / 2);
      hipLaunchKernelGGL(gemm_bf16_kernel<KIND_FWD1>, dim3(nt * max_mt), dim3(NTHR), 0, s, a, nt);
      break;
    }
    case KIND_FWD2: {
      const int nt = (a.H + BN - 1) / BN;
      hipLaunchKernelGGL(gemm_bf16_kernel<KIND_FWD2>, dim3(nt * max_mt), dim3(NTHR), 0, s, a, nt);
      break;
    }
    case KIND_DGRAD2: {
      const int nt = (a.I + BN - 1) / BN;
      hipLaunchKernelGGL(gemm_bf16_kernel<KIND_DGRAD2>, dim3(nt * max_mt), dim3(NTHR), 0, s, a, nt);
      break;
    }
    case KIND_DGRAD1: {
      const int nt = (a.H + BN - 1) / BN;
      hipLaunchKernelGGL(gemm_bf16_kernel<KIND_DGRAD1>, dim3(nt * max_mt), dim3(NTHR), 0, s, a, nt);
      break;
    }
    case KIND_WGRAD2: {
      const int nt = (a.I + BN - 1) / BN, mt = (a.H + BM - 1) / BM;
      hipLaunchKernelGGL(gemm_bf16_kernel<KIND_WGRAD2>, dim3(nt * mt, a.E), dim3(NTHR), 0, s, a, nt);
      break;
    }
    case KIND_WGRAD1: {
      const int nt = (a.H + BN - 1) / BN, mt = (2 * a.I + BM - 1) / BM;
      hipLaunchKernelGGL(gemm_bf16_kernel<KIND_WGRAD1>, dim3(nt * mt, a.E), dim3(NTHR), 0, s, a, nt);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
