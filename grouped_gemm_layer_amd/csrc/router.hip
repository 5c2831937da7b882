// Router projection and its backward (TE dropless-MoE page, "01 Why is MoE
// training harder than dense training?": the router is trained, so it needs
// a gradient; its form is the plain linear one, logits = x W_r^T):
//   forward : logits[t, e] = <x[t], W_r[e]>                       (fp32)
//   backward: dx[t]  += sum_j dlogits[t, idx[t,j]] W_r[idx[t,j]]   (dlogits is
//             zero off the token's top-k set, so these k rows are the whole
//             product dlogits W_r)
//             dW_r[e] = sum over the rows r of expert e (in a fixed order
//             over its sorted rows) of dlogits[t(r), e] x[t(r)]    (fp32)
// x and W_r are bf16.  Everything is deterministic (fixed summation orders,
// no atomics).
#include "moe_internal.h"

namespace moe {
namespace {

// One block of RL_NW waves per 64 tokens x 64 experts, K = H in steps of 32:
// wave w takes the steps w, w + RL_NW, ... and the waves' partial sums are
// added in wave order through LDS (fixed order, fp32).  Operands are read
// straight from global memory into MFMA fragments (the projection is
// 2 T E H flop, a few percent of the layer; its operands stay in L2).  With
// v_mfma_f32_16x16x32_bf16 called as mfma(P, Q, c), lane l holds
// sum_k P[4 (l/16) + v][k] Q[l%16][k], v = 0..3, and an operand fragment is
// row l%16, K elements 8 (l/16) .. +7: here P = W_r rows (experts) and Q = x
// rows (tokens), so a lane ends with 4 consecutive experts of one token.
constexpr int RL_T = 64, RL_E = 64, RL_NW = 4;

__global__ __launch_bounds__(64 * RL_NW) void router_logits_kernel(const bf16_t* __restrict__ x,
                                                                   const bf16_t* __restrict__ wr, int T, int H,
                                                                   int E, float* __restrict__ logits) {
  __shared__ f32x4_t s_acc[RL_NW - 1][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RL_T, e0 = blockIdx.y * RL_E;
  const int r = lane & 15, kq = 8 * (lane >> 4);
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // rows past T or E read row 0 (in bounds) and are never stored
  const bf16_t* xr[4];
  const bf16_t* wrr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * i + r, e = e0 + 16 * i + r;
    xr[i] = x + (size_t)(t < T ? t : 0) * H + kq;
    wrr[i] = wr + (size_t)(e < E ? e : 0) * H + kq;
  }
  for (int k0 = 32 * wave; k0 < H; k0 += 32 * RL_NW) {
    bf16x8_t xf[4], wf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[i] = *reinterpret_cast<const bf16x8_t*>(xr[i] + k0);
      wf[i] = *reinterpret_cast<const bf16x8_t*>(wrr[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)       // token block
#pragma unroll
      for (int j = 0; j < 4; ++j)     // expert block
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_acc[wave - 1][4 * i + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < RL_NW - 1; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += s_acc[w][4 * i + j][lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * i + r;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 16 * j + 4 * (lane >> 4);
      float* dst = logits + (size_t)t * E + e;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (e + v < E) dst[v] = acc[i][j][v];
    }
  }
}

// dx[t] += sum_j dlogits[t, idx[t, j]] * W_r[idx[t, j]], fp32 in slot order
// on top of dx's value, rounded once.  One block per token, 8 columns per
// thread.
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dlogits,
                                                        const int32_t* __restrict__ idx,
                                                        const bf16_t* __restrict__ wr, int k, int H, int E,
                                                        bf16_t* __restrict__ dx) {
  __shared__ int s_e[32];
  __shared__ float s_d[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    const int e = idx[(size_t)t * k + threadIdx.x];
    s_e[threadIdx.x] = e;
    s_d[threadIdx.x] = dlogits[(size_t)t * E + e];
  }
  __syncthreads();
  for (int h0 = threadIdx.x * 8; h0 < H; h0 += 256 * 8) {
    const uint4 d0 = *reinterpret_cast<const uint4*>(dx + (size_t)t * H + h0);
    const uint32_t dw[4] = {d0.x, d0.y, d0.z, d0.w};
    float acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __uint_as_float(dw[i] << 16);
      acc[2 * i + 1] = __uint_as_float(dw[i] & 0xFFFF0000u);
    }
    for (int j0 = 0; j0 < k; j0 += 8) {   // the rows of 8 slots in flight together
      uint4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        w[u] = j0 + u < k ? *reinterpret_cast<const uint4*>(wr + (size_t)s_e[j0 + u] * H + h0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= k) break;
        const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
        const float g = s_d[j0 + u];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += g * __uint_as_float(ww[i] << 16);
          acc[2 * i + 1] += g * __uint_as_float(ww[i] & 0xFFFF0000u);
        }
      }
    }
    *reinterpret_cast<uint4*>(dx + (size_t)t * H + h0) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7]));
  }
}

// dW_r[e][h] for one expert e (blockIdx.y) and 512 columns (8 per lane).
// The expert's sorted rows go in batches of RDW_RB: batch b belongs to wave
// b % RDW_NW, which sums its batches in order and each batch's rows in order;
// the waves' partial sums are then added in wave order through LDS (fixed
// order, fp32).  Per batch, lanes 0..RDW_RB-1 load the rows' token indices and
// dlogits in one instruction each, and all RDW_RB x rows are in flight
// together.  An expert with no rows writes zeros.
constexpr int RDW_COLS = 512, RDW_NW = 8, RDW_RB = 16;

__global__ __launch_bounds__(64 * RDW_NW) void router_dw_kernel(const float* __restrict__ dlogits,
                                                                const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ s2f,
                                                                const bf16_t* __restrict__ x, int k, int H, int E,
                                                                float* __restrict__ dwr) {
  __shared__ __attribute__((aligned(16))) float s_part[RDW_NW - 1][RDW_COLS];
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h0 = blockIdx.x * RDW_COLS + 8 * lane;
  const bool live = h0 < H;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int rb = r0 + wave * RDW_RB; rb < r1; rb += RDW_NW * RDW_RB) {
    const int rr = rb + (lane & (RDW_RB - 1));
    const int tl = rr < r1 ? s2f[rr] / k : -1;            // lane u < RDW_RB: token of row rb + u
    const float dl = tl >= 0 ? dlogits[(size_t)tl * E + e] : 0.f;
    uint4 v[RDW_RB];
#pragma unroll
    for (int u = 0; u < RDW_RB; ++u) {
      const int t = __builtin_amdgcn_readlane(tl, u);
      v[u] = (t >= 0 && live) ? *reinterpret_cast<const uint4*>(x + (size_t)t * H + h0) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < RDW_RB; ++u) {
      const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dl), u));
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += d * __uint_as_float(w[i] << 16);
        acc[2 * i + 1] += d * __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s_part[wave - 1][8 * lane + i] = acc[i];
  }
  __syncthreads();
  if (wave == 0 && live) {
#pragma unroll
    for (int w = 0; w < RDW_NW - 1; ++w)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += s_part[w][8 * lane + i];
    float* dst = dwr + (size_t)e * H + h0;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
}

}  // namespace

hipError_t launch_router_logits(const bf16_t* x, const bf16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t s) {
  return launch_kernel(router_logits_kernel, dim3((T + RL_T - 1) / RL_T, (E + RL_E - 1) / RL_E), dim3(64 * RL_NW), 0,
                       s, x, wr, T, H, E, logits);
}

hipError_t launch_router_project_bwd(const float* dlogits, const int32_t* topk_idx, const int32_t* offsets,
                                     const int32_t* s2f, const bf16_t* x, const bf16_t* wr, int T, int H, int E,
                                     int k, bf16_t* dx, float* dwr, hipStream_t s) {
  const hipError_t e = launch_kernel(router_dx_kernel, dim3(T), dim3(256), 0, s, dlogits, topk_idx, wr, k, H, E, dx);
  if (e != hipSuccess) return e;
  return launch_kernel(router_dw_kernel, dim3((H + RDW_COLS - 1) / RDW_COLS, E), dim3(64 * RDW_NW), 0, s, dlogits,
                       offsets, s2f, x, k, H, E, dwr);
}

}  // namespace moe
