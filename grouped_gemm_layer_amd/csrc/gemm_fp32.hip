// fp32 grouped GEMMs of the MoE layer (MOE_MODE_FP32): the same six GEMM
// kinds and fused epilogues as the bf16 MFMA path, on plain fp32 FMAs with
// 64x64 LDS tiles.  Meant for tiny shapes and tight-tolerance checks, not
// speed.  See gemm_bf16.hip for the definition of each kind.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = FP32_BM;   // 64
constexpr int BN = FP32_BN;   // 64
constexpr int BK = 16;

template <int KIND>
__global__ __launch_bounds__(256) void gemm_fp32_kernel(LayerArgs a, int n_tiles) {
  constexpr bool ragged_rows = KIND <= KIND_DGRAD1;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  __shared__ float sC[BM][BN + 1];
  const int tid = threadIdx.x;
  const int H = a.H, I = a.I, k = a.k;

  int e, m0, mlim, n0, klo = 0, khi = 0, K;
  if constexpr (ragged_rows) {
    const int nt = blockIdx.x % n_tiles, mt = blockIdx.x / n_tiles;
    e = a.tile_expert[mt];
    if (e < 0) return;
    m0 = a.tile_row0[mt];
    mlim = a.offsets[e + 1];
    n0 = nt * (KIND == KIND_FWD1 ? BN / 2 : BN);
    K = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2) ? H : (KIND == KIND_FWD2 ? I : 2 * I);
  } else {
    e = blockIdx.y;
    const int nt = blockIdx.x % n_tiles, mt = blockIdx.x / n_tiles;
    m0 = mt * BM;
    n0 = nt * BN;
    klo = a.offsets[e];
    khi = a.offsets[e + 1];
    K = khi - klo;
    mlim = (KIND == KIND_WGRAD2) ? H : 2 * I;
  }
  const int nlim = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2 || KIND == KIND_WGRAD2) ? I : H;

  const float* x = static_cast<const float*>(a.x);
  const float* dy = static_cast<const float*>(a.dy);
  const float* w13 = static_cast<const float*>(a.w13) + (size_t)e * 2 * I * H;
  const float* w2 = static_cast<const float*>(a.w2) + (size_t)e * H * I;
  const float* Abuf = static_cast<const float*>(a.A);
  const float* dG13 = static_cast<const float*>(a.dG13);
  const float* Ag = static_cast<const float*>(a.Ag);

  // element accessors (0 outside the valid range)
  auto A_at = [&](int mm, int kk) -> float {
    const int m = m0 + mm;
    if (m >= mlim) return 0.f;
    if constexpr (KIND == KIND_FWD1) return x[(size_t)(a.s2f[m] / k) * H + kk];
    else if constexpr (KIND == KIND_FWD2) return Abuf[(size_t)m * I + kk];
    else if constexpr (KIND == KIND_DGRAD2) return dy[(size_t)(a.s2f[m] / k) * H + kk];
    else if constexpr (KIND == KIND_DGRAD1) return dG13[(size_t)m * 2 * I + kk];
    else {
      const int r = klo + kk;
      if (r >= khi) return 0.f;
      if constexpr (KIND == KIND_WGRAD2) return dy[(size_t)(a.s2f[r] / k) * H + m];
      else return dG13[(size_t)r * 2 * I + m];
    }
  };
  auto B_at = [&](int nn, int kk) -> float {
    if constexpr (KIND == KIND_FWD1) {
      const int c = n0 + (nn & (BN / 2 - 1));
      if (c >= I) return 0.f;
      return w13[(size_t)((nn < BN / 2) ? c : I + c) * H + kk];
    } else {
      const int n = n0 + nn;
      if (n >= nlim) return 0.f;
      if constexpr (KIND == KIND_FWD2) return w2[(size_t)n * I + kk];
      else if constexpr (KIND == KIND_DGRAD2) return w2[(size_t)kk * I + n];
      else if constexpr (KIND == KIND_DGRAD1) return w13[(size_t)kk * H + n];
      else {
        const int r = klo + kk;
        if (r >= khi) return 0.f;
        if constexpr (KIND == KIND_WGRAD2) return Ag[(size_t)r * I + n];
        else return x[(size_t)(a.s2f[r] / k) * H + n];
      }
    }
  };

  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int i = tid; i < BM * BK; i += 256) {
      const int mm = i / BK, kk = i % BK;
      sA[kk][mm] = (k0 + kk < K) ? A_at(mm, k0 + kk) : 0.f;
      sB[kk][mm] = (k0 + kk < K) ? B_at(mm, k0 + kk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = sA[kk][ty * 4 + i]; bv[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) sC[ty * 4 + i][tx * 4 + j] = acc[i][j];
  __syncthreads();

  if constexpr (KIND == KIND_FWD1) {
    float* G13 = static_cast<float*>(a.G13);
    float* Aout = static_cast<float*>(a.A);
    for (int i = tid; i < BM * (BN / 2); i += 256) {
      const int mm = i / (BN / 2), c = i % (BN / 2);
      const int m = m0 + mm, col = n0 + c;
      if (m >= mlim || col >= I) continue;
      const float g1 = sC[mm][c], g3 = sC[mm][BN / 2 + c];
      if (G13 != nullptr) {   // none when the forward keeps no state for a backward
        G13[(size_t)m * 2 * I + col] = g1;
        G13[(size_t)m * 2 * I + I + col] = g3;
      }
      if (Aout != nullptr) Aout[(size_t)m * I + col] = g1 * sigmoid_f32(g1) * g3;   // none in the recompute
    }
  } else if constexpr (KIND == KIND_FWD2 || KIND == KIND_DGRAD1) {
    float* out = static_cast<float*>(KIND == KIND_FWD2 ? a.O : a.dXp);
    for (int i = tid; i < BM * BN; i += 256) {
      const int mm = i / BN, nn = i % BN;
      const int m = m0 + mm, n = n0 + nn;
      if (m < mlim && n < nlim) out[(size_t)m * H + n] = sC[mm][nn];
    }
  } else if constexpr (KIND == KIND_DGRAD2) {
    const float* G13 = static_cast<const float*>(a.G13);
    float* dG = static_cast<float*>(a.dG13);
    float* Agw = static_cast<float*>(a.Ag);
    for (int i = tid; i < BM * BN; i += 256) {
      const int mm = i / BN, nn = i % BN;
      const int m = m0 + mm, n = n0 + nn;
      if (m >= mlim || n >= I) continue;
      const float g = a.gate[a.s2f[m]];
      const float g1 = G13[(size_t)m * 2 * I + n], g3 = G13[(size_t)m * 2 * I + I + n];
      const float s = sigmoid_f32(g1), silu = g1 * s;
      const float da = g * sC[mm][nn];
      dG[(size_t)m * 2 * I + n] = da * g3 * s * (1.f + g1 * (1.f - s));
      dG[(size_t)m * 2 * I + I + n] = da * silu;
      Agw[(size_t)m * I + n] = g * silu * g3;
    }
    if (tid < BM) {
      const int m = m0 + tid;
      if (m < mlim) {
        float p = 0.f;
        for (int nn = 0; nn < BN && n0 + nn < I; ++nn) {
          const int n = n0 + nn;
          const float g1 = G13[(size_t)m * 2 * I + n], g3 = G13[(size_t)m * 2 * I + I + n];
          p += sC[tid][nn] * (g1 * sigmoid_f32(g1) * g3);
        }
        a.dgate_part[(size_t)(n0 / BN) * a.M + m] = p;
      }
    }
  } else {
    float* out = (KIND == KIND_WGRAD2) ? a.dw2 + (size_t)e * H * I : a.dw13 + (size_t)e * 2 * I * H;
    const int ld = (KIND == KIND_WGRAD2) ? I : H;
    for (int i = tid; i < BM * BN; i += 256) {
      const int mm = i / BN, nn = i % BN;
      const int m = m0 + mm, n = n0 + nn;
      if (m < mlim && n < nlim) out[(size_t)m * ld + n] = a.wgrad_acc ? out[(size_t)m * ld + n] + sC[mm][nn] : sC[mm][nn];
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp32(GemmKind kind, const LayerArgs& a, hipStream_t s) {
  const int max_mt = max_row_tiles(a.M, a.E, BM);
  switch (kind) {
    case KIND_FWD1: {
      const int nt = (a.I + BN / 2 - 1) / (BN / 2);
      return launch_kernel(gemm_fp32_kernel<KIND_FWD1>, dim3(nt * max_mt), dim3(256), 0, s, a, nt);
    }
    case KIND_FWD2: {
      const int nt = (a.H + BN - 1) / BN;
      return launch_kernel(gemm_fp32_kernel<KIND_FWD2>, dim3(nt * max_mt), dim3(256), 0, s, a, nt);
    }
    case KIND_DGRAD2: {
      const int nt = (a.I + BN - 1) / BN;
      return launch_kernel(gemm_fp32_kernel<KIND_DGRAD2>, dim3(nt * max_mt), dim3(256), 0, s, a, nt);
    }
    case KIND_DGRAD1: {
      const int nt = (a.H + BN - 1) / BN;
      return launch_kernel(gemm_fp32_kernel<KIND_DGRAD1>, dim3(nt * max_mt), dim3(256), 0, s, a, nt);
    }
    case KIND_WGRAD2: {
      const int nt = (a.I + BN - 1) / BN, mt = (a.H + BM - 1) / BM;
      return launch_kernel(gemm_fp32_kernel<KIND_WGRAD2>, dim3(nt * mt, a.E), dim3(256), 0, s, a, nt);
    }
    case KIND_WGRAD1: {
      const int nt = (a.H + BN - 1) / BN, mt = (2 * a.I + BM - 1) / BM;
      return launch_kernel(gemm_fp32_kernel<KIND_WGRAD1>, dim3(nt * mt, a.E), dim3(256), 0, s, a, nt);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
