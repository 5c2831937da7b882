// Combine (forward) and unpermute-reduce (backward), and the router backward.
//
// Combine returns the expert rows to token order and sums the results of the
// token's experts (TE dropless-MoE page, "Optimisation 2: dispatch and combine
// via NCCL EP"), here weighted by the gates:
//   out[t] = sum_{j=0..k-1} gate[t,j] * rows[f2s[t*k+j]]    (fp32, slot order)
// With gate == nullptr the weights are 1 (the backward's dX reduction).
// One block per token, 16-byte vectors per thread: HBM-bound row traffic,
// deterministic (no atomics).
#include "moe_internal.h"

// Row loads (1) and output stores (2) non-temporal: every row is read once,
// so caching it only evicts other data (combine 0.123 -> 0.099 ms,
// unpermute-reduce 0.119 -> 0.100 at the 30B shape; 0 = plain accesses).
#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 2
#endif

namespace moe {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));   // 16 bytes

template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> { static constexpr int N = 8; };
template <> struct Vec16<float> { static constexpr int N = 4; };

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ rows, const int32_t* __restrict__ f2s,
                                                      const float* __restrict__ gate, int k, int H,
                                                      T* __restrict__ out) {
  constexpr int V = Vec16<T>::N;
  __shared__ int s_row[32];
  __shared__ float s_g[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = f2s[(size_t)t * k + threadIdx.x];
    s_g[threadIdx.x] = gate ? gate[(size_t)t * k + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  for (int h0 = threadIdx.x * V; h0 < H; h0 += 256 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
#if MOE_COMBINE_NT >= 1
      const u32x4v raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(rows + (size_t)s_row[j] * H + h0));
#else
      const u32x4v raw = *reinterpret_cast<const u32x4v*>(rows + (size_t)s_row[j] * H + h0);
#endif
      const float g = s_g[j];
      if constexpr (V == 8) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += g * __uint_as_float(w[i] << 16);
          acc[2 * i + 1] += g * __uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else {
        acc[0] += g * __uint_as_float(raw.x);
        acc[1] += g * __uint_as_float(raw.y);
        acc[2] += g * __uint_as_float(raw.z);
        acc[3] += g * __uint_as_float(raw.w);
      }
    }
    u32x4v o;
    if constexpr (V == 8) {
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
    } else {
      o.x = __float_as_uint(acc[0]);
      o.y = __float_as_uint(acc[1]);
      o.z = __float_as_uint(acc[2]);
      o.w = __float_as_uint(acc[3]);
    }
#if MOE_COMBINE_NT >= 2
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4v*>(out + (size_t)t * H + h0));
#else
    *reinterpret_cast<u32x4v*>(out + (size_t)t * H + h0) = o;
#endif
  }
}

template <typename T>
hipError_t launch_combine(const T* rows, const int32_t* f2s, const float* gate, int Tn, int k, int H, T* out,
                          hipStream_t s) {
  return launch_kernel(combine_kernel<T>, dim3(Tn), dim3(256), 0, s, rows, f2s, gate, k, H, out);
}
template hipError_t launch_combine<bf16_t>(const bf16_t*, const int32_t*, const float*, int, int, int, bf16_t*,
                                           hipStream_t);
template hipError_t launch_combine<float>(const float*, const int32_t*, const float*, int, int, int, float*,
                                          hipStream_t);

// Router backward, one wave per token:
//   dgate[t,j] = sum_p dgate_part[p][row of slot j]      (p ascending)
//   dlogits[t,e] = gate_j (dgate_j - sum_i gate_i dgate_i) if e = idx[t,j], else 0
// (softmax over the selected logits, differentiated).
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ part, int n_parts,
                                                         const int32_t* __restrict__ f2s,
                                                         const float* __restrict__ gate,
                                                         const int32_t* __restrict__ idx, int Tn, int k, int E,
                                                         int M, float* __restrict__ dgate,
                                                         float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  float dg = 0.f, g = 0.f;
  int e = -1;
  if (lane < k) {
    const size_t f = (size_t)t * k + lane;
    const int r = f2s[f];
    for (int p0 = 0; p0 < n_parts; p0 += 4) {   // the partials of 4 column tiles in flight together
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = p0 + u < n_parts ? part[(size_t)(p0 + u) * M + r] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) dg += v[u];                  // p ascending
    }
    g = gate[f];
    e = idx[f];
    dgate[f] = dg;
  }
  float inner = g * dg;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) inner += __shfl_xor(inner, off);
  if (dlogits == nullptr) return;
  const float mine = g * (dg - inner);
  float* row = dlogits + (size_t)t * E;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int ee = e0 + lane;
    float val = 0.f;
    for (int j = 0; j < k; ++j) {   // slot j's expert and value, read as scalars from lane j
      const int ej = __builtin_amdgcn_readlane(e, j);
      const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), j));
      if (ej == ee) val = vj;
    }
    if (ee < E) row[ee] = val;
  }
}

hipError_t launch_router_bwd(const float* dgate_part, int n_parts, const int32_t* f2s, const float* gate,
                             const int32_t* topk_idx, int Tn, int k, int E, int M, float* dgate, float* dlogits,
                             hipStream_t s) {
  return launch_kernel(router_bwd_kernel, dim3((Tn + 3) / 4), dim3(256), 0, s, dgate_part, n_parts, f2s, gate,
                     topk_idx, Tn, k, E, M, dgate, dlogits);
}

// Split-K completion of the weight gradients: for each expert whose rows were
// split into chunks (its rank r has cstart[r+1] - cstart[r] > 1 chunks; they
// are the first ranks, the work list being ordered by decreasing row count),
// dW[e] = chunk 0's result (already in dW) + the partial slots of chunks
// 1, 2, ... added in that order, elementwise in fp32 -- deterministic, no
// atomics.  blockIdx.y = rank, blockIdx.z = matrix (0: dW13, 1: dW2).
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const int32_t* __restrict__ order,
                                                           const int32_t* __restrict__ cstart,
                                                           const int32_t* __restrict__ slot0,
                                                           float* __restrict__ dw13, const float* __restrict__ p13,
                                                           size_t n13, float* __restrict__ dw2,
                                                           const float* __restrict__ p2, size_t n2) {
  const int r = blockIdx.y;
  const int nch = cstart[r + 1] - cstart[r];
  if (nch <= 1) return;
  const bool w13 = blockIdx.z == 0;
  const size_t n = w13 ? n13 : n2;
  float* dw = (w13 ? dw13 : dw2) + (size_t)order[r] * n;
  const float* p = (w13 ? p13 : p2) + (size_t)slot0[r] * n;
  constexpr int U = 4;                     // 16-byte vectors per thread per pass
  const size_t step = (size_t)gridDim.x * 256 * 4 * U;
  for (size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i0 < n; i0 += step) {
    f32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + (size_t)u * gridDim.x * 256 * 4;
      v[u] = i < n ? *reinterpret_cast<const f32x4_t*>(dw + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int c = 1; c < nch; ++c) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = i0 + (size_t)u * gridDim.x * 256 * 4;
        if (i < n) v[u] += *reinterpret_cast<const f32x4_t*>(p + (size_t)(c - 1) * n + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + (size_t)u * gridDim.x * 256 * 4;
      if (i < n) *reinterpret_cast<f32x4_t*>(dw + i) = v[u];
    }
  }
}

hipError_t launch_wgrad_reduce(const LayerArgs& a, hipStream_t s) {
  const int ranks = max(1, min(a.E, (int)wgrad_max_slots((size_t)a.M)));   // split experts come first
  const size_t n13 = (size_t)2 * a.I * a.H, n2 = (size_t)a.H * a.I;
  return launch_kernel(wgrad_reduce_kernel, dim3(128, ranks, 2), dim3(256), 0, s, a.wg_order, a.wg_cstart,
                     a.wg_slot0, a.dw13, a.wpart13, n13, a.dw2, a.wpart2, n2);
}

}  // namespace moe
