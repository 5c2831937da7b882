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
// operand's GEMM-K (contiguous).  The scaling by 2^-X and the rounding are
// exact in fp32, so the codes equal those of the exact definition for the
// same bf16 inputs.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int ea;
  const float m = frexpf(amax, &ea);   // amax = m 2^ea, m in [0.5, 1)
  // amax = (2m) 2^(ea-1); 448 = 1.75 2^8
  const int X = (2.f * m <= 1.75f) ? ea - 9 : ea - 8;
  return min(max(X, -127), 127);
}

__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.f);
  uint32_t code;
  if (a < 0.015625f) {                 // below 2^-6: subnormal grid m 2^-9, m = 0..8
    code = (uint32_t)rintf(a * 512.f); // m = 8 is 2^-6, the smallest normal (code 0x08)
  } else {
    int e;
    (void)frexpf(a, &e);
    int E = e - 1;                     // a in [2^E, 2^(E+1)), E >= -6
    uint32_t q = (uint32_t)rintf(ldexpf(a, 3 - E));   // 8..16, exact scaling, ties to even
    if (q == 16u) { q = 8u; E += 1; }
    code = min(((uint32_t)(E + 7) << 3) | (q - 8u), 0x7Eu);
  }
  return code | sign;
}

// 32 values -> 32 codes packed into 8 words, returns the E8M0 byte.
__device__ __forceinline__ uint32_t mx_quant_block(const float (&v)[32], uint32_t (&packed)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_scale_exp(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= e4m3_encode(ldexpf(v[4 * w + b], -X)) << (8 * b);
    packed[w] = word;
  }
  return (uint32_t)(X + 127);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 r, float* out) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// 32 consecutive elements of a row, bf16 or fp32
__device__ __forceinline__ void load32(const bf16_t* p, float (&v)[32]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack_bf16x8(q[i], v + 8 * i);
}
__device__ __forceinline__ void load32(const float* p, float (&v)[32]) {
  const f32x4_t* q = reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4_t w = q[i];
    v[4 * i] = w[0]; v[4 * i + 1] = w[1]; v[4 * i + 2] = w[2]; v[4 * i + 3] = w[3];
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

// Column blocks, per expert: source S[e] is [Kd][N] (K outer); output codes
// [e][N][Kd] (K contiguous) and scales [e][N][Kd/32].  Thread = one column n
// and MX_KTILE consecutive k (4 blocks): the loads of one source row are
// contiguous across the threads, each thread stores one 128-byte line.
__global__ __launch_bounds__(256) void mx_quant_cols_t_kernel(const bf16_t* __restrict__ src, int Kd, int N,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y, e = blockIdx.z;
  if (n >= N) return;
  const bf16_t* s = src + (size_t)e * Kd * N + (size_t)(MX_KTILE * c) * N + n;
  uint4* o = reinterpret_cast<uint4*>(codes + ((size_t)e * N + n) * Kd + MX_KTILE * c);
  uint32_t sc4 = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(s[(size_t)(32 * q + i) * N]);
    uint32_t packed[8];
    sc4 |= mx_quant_block(v, packed) << (8 * q);
    o[2 * q] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    o[2 * q + 1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
  *reinterpret_cast<uint32_t*>(scales + ((size_t)e * N + n) * (Kd / 32) + 4 * c) = sc4;
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

// Token blocks, transposed: source rows r (expert-sorted order) of a [.][F]
// matrix, read as src[s2f[r] / k] when s2f is given (gathered x / dY rows);
// output codes [F][Mp] and scales [F][Mp/32].  Block = one padded tile of
// MX_KTILE tokens (inside a single expert's padded range) x 256 features;
// thread = one feature, 4 blocks of 32 tokens, one 128-byte line of codes.
template <typename T>
__global__ __launch_bounds__(256) void mx_quant_tokens_t_kernel(const T* __restrict__ src, int F,
                                                                const int32_t* __restrict__ s2f, int k,
                                                                const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ pad_off, int E,
                                                                int Mp, uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  __shared__ int s_src[MX_KTILE];       // source row of each token of the tile, -1 = padding
  const int p0 = MX_KTILE * blockIdx.y;
  if (p0 >= pad_off[E]) return;         // uniform over the block
  int lo = 0, hi = E - 1;               // expert e with pad_off[e] <= p0 < pad_off[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pad_off[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  if (threadIdx.x < MX_KTILE) {
    const int r = offsets[e] + (p0 - pad_off[e]) + threadIdx.x;
    s_src[threadIdx.x] = (r < offsets[e + 1]) ? (s2f ? s2f[r] / k : r) : -1;
  }
  __syncthreads();
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  uint4* o = reinterpret_cast<uint4*>(codes + (size_t)f * Mp + p0);
  uint32_t sc4 = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int sr = s_src[32 * q + t];
      v[t] = (sr >= 0) ? ElemTraits<T>::load(src + (size_t)sr * F + f) : 0.f;
    }
    uint32_t packed[8];
    sc4 |= mx_quant_block(v, packed) << (8 * q);
    o[2 * q] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    o[2 * q + 1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
  *reinterpret_cast<uint32_t*>(scales + (size_t)f * (Mp / 32) + p0 / 32) = sc4;
}

template <typename T>
hipError_t launch_mx_quant_rows(const T* src, int R, int K, const int32_t* s2f, int k, uint8_t* codes,
                                uint8_t* scales, hipStream_t s) {
  const long total = (long)R * (K / 32);
  const int grid = (int)min((total + 255) / 256, (long)65536);
  hipLaunchKernelGGL(mx_quant_rows_kernel<T>, dim3(grid), dim3(256), 0, s, src, R, K, s2f, k, codes, scales);
  return hipGetLastError();
}
template hipError_t launch_mx_quant_rows<bf16_t>(const bf16_t*, int, int, const int32_t*, int, uint8_t*, uint8_t*,
                                                 hipStream_t);
template hipError_t launch_mx_quant_rows<float>(const float*, int, int, const int32_t*, int, uint8_t*, uint8_t*,
                                                hipStream_t);

hipError_t launch_mx_quant_cols_t(const bf16_t* src, int E, int Kd, int N, uint8_t* codes, uint8_t* scales,
                                  hipStream_t s) {
  hipLaunchKernelGGL(mx_quant_cols_t_kernel, dim3((N + 255) / 256, Kd / MX_KTILE, E), dim3(256), 0, s, src, Kd, N,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* pad_off, hipStream_t s) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(512), 0, s, offsets, E, pad_off);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mx_quant_tokens_t(const T* src, int F, const int32_t* s2f, int k, const int32_t* offsets,
                                    const int32_t* pad_off, int E, int Mp, uint8_t* codes, uint8_t* scales,
                                    hipStream_t s) {
  hipLaunchKernelGGL(mx_quant_tokens_t_kernel<T>, dim3((F + 255) / 256, Mp / MX_KTILE), dim3(256), 0, s, src, F,
                     s2f, k, offsets, pad_off, E, Mp, codes, scales);
  return hipGetLastError();
}
template hipError_t launch_mx_quant_tokens_t<bf16_t>(const bf16_t*, int, const int32_t*, int, const int32_t*,
                                                     const int32_t*, int, int, uint8_t*, uint8_t*, hipStream_t);
template hipError_t launch_mx_quant_tokens_t<float>(const float*, int, const int32_t*, int, const int32_t*,
                                                    const int32_t*, int, int, uint8_t*, uint8_t*, hipStream_t);

}  // namespace moe
