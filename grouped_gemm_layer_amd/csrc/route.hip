// Routing kernels: top-k + gates, expert histogram, expert-major scan, stable
// scatter into the expert-sorted order, and the ragged tile table.
//
// What is computed (TE dropless-MoE page, "01" and "03": the router assigns
// each token to a few experts and every token is kept; "Optimisation 1": the
// per-expert token counts stay on the device):
//   idx[t, j]  = j-th largest logit of token t, key (-logit, expert id)
//   gate[t, j] = softmax over the k selected logits
//   counts, offsets, and the stable sort of flat slots t*k+j by expert.
// All integer results are bit-exact and independent of scheduling: LDS
// atomics only count (order-free), and ranks come from wave ballots.
#include "moe_internal.h"

#include <math.h>

#include <mutex>

namespace moe {

constexpr int ROUTE_CHUNK = 4096;   // flat slots per block of the histogram / scatter
constexpr int MAX_EPL = 8;          // logits per lane: E <= 512
constexpr int MAX_E = 512;

int route_num_blocks(int M) { return (M + ROUTE_CHUNK - 1) / ROUTE_CHUNK; }

// (value, expert) of the better entry: larger value, then smaller expert id;
// id INT_MAX marks "no entry"
__device__ __forceinline__ void take_better(float ov, int oe, float& bv, int& be) {
  if (oe != INT_MAX && (be == INT_MAX || ov > bv || (ov == bv && oe < be))) { bv = ov; be = oe; }
}
// one cross-lane step of the wave arg-max through DPP (lanes paired inside rows of 16)
template <int CTRL>
__device__ __forceinline__ void best_dpp(float& bv, int& be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  take_better(ov, oe, bv, be);
}
// one cross-lane step through a gfx950 row swap (rows 0-1 and 2-3 for 16,
// the two halves for 32): the swap returns each lane its own and its
// partner's word, in the same order for the value and the expert
template <int ROWS>
__device__ __forceinline__ void best_swap(float& bv, int& be) {
  const auto swap = [](uint32_t w) {
    if constexpr (ROWS == 16) return __builtin_amdgcn_permlane16_swap(w, w, false, false);
    else return __builtin_amdgcn_permlane32_swap(w, w, false, false);
  };
  const auto rv = swap(__float_as_uint(bv));
  const auto re = swap((uint32_t)be);
  float v = __uint_as_float(rv[0]);
  int e = (int)re[0];
  take_better(__uint_as_float(rv[1]), (int)re[1], v, e);
  bv = v;
  be = e;
}

// One wave per token, four tokens per block.  Each of the k rounds takes the
// best remaining entry of every lane, then the wave's best through six
// cross-lane steps (quad swaps, the two row mirrors, the row swaps), after
// which every lane holds the same (value, expert): the order of the
// comparisons does not change the result, the key being a strict order.
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ logits, int T, int E,
                                                        int k, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole waves leave; no block barrier follows
  const float* row = logits + (size_t)t * E;
  float v[MAX_EPL];
  uint32_t live = 0;
#pragma unroll
  for (int q = 0; q < MAX_EPL; ++q) {
    const int e = lane + 64 * q;
    v[q] = 0.f;
    if (e < E) { v[q] = row[e]; live |= 1u << q; }
  }
  float my_v = 0.f, v0 = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    // best (largest value, then smallest id) among this lane's live entries
    float bv = 0.f;
    int be = INT_MAX;
#pragma unroll
    for (int q = 0; q < MAX_EPL; ++q)
      if (live & (1u << q)) take_better(v[q], lane + 64 * q, bv, be);
    best_dpp<0xB1>(bv, be);    // quad_perm 1,0,3,2
    best_dpp<0x4E>(bv, be);    // quad_perm 2,3,0,1
    best_dpp<0x141>(bv, be);   // row_half_mirror
    best_dpp<0x140>(bv, be);   // row_mirror
    best_swap<16>(bv, be);
    best_swap<32>(bv, be);
    if (lane == (be & 63)) live &= ~(1u << (be >> 6));
    if (j == 0) v0 = bv;
    if (lane == j) { my_v = bv; my_e = be; }
  }
  float ex = (lane < k) ? expf(my_v - v0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    gate[(size_t)t * k + lane] = ex / sum;
  }
}

// k <= 8: four lanes per token, 64 tokens per block.  Lane q of a token scans
// experts [q E/4, (q+1) E/4) in ascending order and keeps the 8 best (value,
// expert) pairs sorted in registers: a new value enters before the first slot
// it beats strictly, so an equal value with a larger id stays behind (the key
// (-logit, id)).  Then the lists of lanes q and q^1, and of q and q^2, merge
// through DPP quad swaps, the higher lane's pairs (all with larger ids)
// inserted into the lower lane's list by the same rule; lane 0 of the quad
// ends with the token's top k, in order, and its softmax gates.
constexpr int TOPK_SMALL = 8;
__device__ __forceinline__ void topk_insert(float x, int id, float (&v)[TOPK_SMALL], int (&ix)[TOPK_SMALL]) {
  // slot j becomes: itself if x does not beat it, x if x beats it but not
  // slot j - 1, else the old slot j - 1 (shifted down); from the last slot up
#pragma unroll
  for (int j = TOPK_SMALL - 1; j >= 0; --j) {
    const bool c = x > v[j];
    const bool cp = j > 0 && x > v[j > 0 ? j - 1 : 0];
    const float nv = cp ? v[j > 0 ? j - 1 : 0] : x;
    const int ni = cp ? ix[j > 0 ? j - 1 : 0] : id;
    v[j] = c ? nv : v[j];
    ix[j] = c ? ni : ix[j];
  }
}
template <int CTRL>
__device__ __forceinline__ void topk_merge(float (&v)[TOPK_SMALL], int (&ix)[TOPK_SMALL], bool lower) {
  float pv[TOPK_SMALL];
  int pi[TOPK_SMALL];
#pragma unroll
  for (int j = 0; j < TOPK_SMALL; ++j) {
    pv[j] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[j]), CTRL, 0xF, 0xF, false));
    pi[j] = __builtin_amdgcn_update_dpp(0, ix[j], CTRL, 0xF, 0xF, false);
  }
  if (lower) {
#pragma unroll
    for (int j = 0; j < TOPK_SMALL; ++j) topk_insert(pv[j], pi[j], v, ix);
  }
}
__global__ __launch_bounds__(256) void topk_gate_small_kernel(const float* __restrict__ logits, int T, int E,
                                                              int k, int32_t* __restrict__ idx,
                                                              float* __restrict__ gate) {
  const int q = threadIdx.x & 3;
  const int t = blockIdx.x * 64 + (threadIdx.x >> 2);
  const bool live = t < T;     // no early exit: the merges read the whole quad
  float v[TOPK_SMALL];
  int ix[TOPK_SMALL];
#pragma unroll
  for (int j = 0; j < TOPK_SMALL; ++j) {
    v[j] = -INFINITY;
    ix[j] = INT_MAX;
  }
  const int per = (E + 3) / 4;
  const int e0 = min(E, q * per), e1 = min(E, e0 + per);
  if (live) {
    const float* row = logits + (size_t)t * E;
    if ((E & 3) == 0 && (per & 3) == 0) {   // 16-byte aligned quarters
      for (int e = e0; e < e1; e += 4) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(row + e);
        topk_insert(x[0], e, v, ix);
        topk_insert(x[1], e + 1, v, ix);
        topk_insert(x[2], e + 2, v, ix);
        topk_insert(x[3], e + 3, v, ix);
      }
    } else {
      for (int e = e0; e < e1; ++e) topk_insert(row[e], e, v, ix);
    }
  }
  topk_merge<0xB1>(v, ix, (q & 1) == 0);   // quad_perm 1,0,3,2: lanes q, q^1
  topk_merge<0x4E>(v, ix, (q & 2) == 0);   // quad_perm 2,3,0,1: lanes q, q^2
  if (live && q == 0) {
    float ex[TOPK_SMALL], sum = 0.f;
#pragma unroll
    for (int j = 0; j < TOPK_SMALL; ++j) {
      ex[j] = j < k ? expf(v[j] - v[0]) : 0.f;
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < TOPK_SMALL; ++j)
      if (j < k) {
        idx[(size_t)t * k + j] = ix[j];
        gate[(size_t)t * k + j] = ex[j] / sum;
      }
  }
}

// Per-block expert histogram of ROUTE_CHUNK flat slots (1024 threads).
constexpr int ROUTE_THREADS = 1024;   // threads of the histogram and scatter blocks
__global__ __launch_bounds__(ROUTE_THREADS) void expert_hist_kernel(const int32_t* __restrict__ idx, int M, int E,
                                                                    int32_t* __restrict__ partials) {
  __shared__ int s_hist[MAX_E];
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) s_hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * ROUTE_CHUNK;
  for (int i = threadIdx.x; i < ROUTE_CHUNK; i += ROUTE_THREADS) {
    const int f = base + i;
    if (f < M) atomicAdd(&s_hist[idx[f]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) partials[blockIdx.x * E + e] = s_hist[e];
}

// One block: counts, offsets and the expert-major block bases
//   bases[b][e] = offsets[e] + sum_{b' < b} partials[b'][e].
// Each thread (expert) reads its column of partials SCAN_U blocks at a time,
// so the loads of a batch are in flight together.
constexpr int SCAN_U = 16;
__global__ __launch_bounds__(1024) void expert_scan_kernel(const int32_t* __restrict__ partials, int nblk,
                                                           int E, int32_t* __restrict__ bases,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int s_scan[2][MAX_E];
  const int e = threadIdx.x;
  auto load_batch = [&](int b0, int (&c)[SCAN_U]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SCAN_U; ++u) c[u] = (b0 + u < nblk) ? partials[(size_t)(b0 + u) * E + e] : 0;
  };
  int run = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nblk; b0 += SCAN_U) {
      int c[SCAN_U];
      load_batch(b0, c);
#pragma unroll
      for (int u = 0; u < SCAN_U; ++u) run += c[u];
    }
    counts[e] = run;
  }
  // inclusive Hillis-Steele scan over experts
  int cur = 0;
  if (e < MAX_E) s_scan[0][e] = (e < E) ? run : 0;
  __syncthreads();
  for (int off = 1; off < MAX_E; off <<= 1) {
    if (e < MAX_E) {
      int val = s_scan[cur][e];
      if (e >= off) val += s_scan[cur][e - off];
      s_scan[cur ^ 1][e] = val;
    }
    cur ^= 1;
    __syncthreads();
  }
  if (e < E) {
    const int excl = s_scan[cur][e] - run;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = s_scan[cur][e];
    int pre = excl;
    for (int b0 = 0; b0 < nblk; b0 += SCAN_U) {
      int c[SCAN_U];
      load_batch(b0, c);
#pragma unroll
      for (int u = 0; u < SCAN_U; ++u) {
        if (b0 + u < nblk) bases[(size_t)(b0 + u) * E + e] = pre;
        pre += c[u];
      }
    }
  }
}

// Stable scatter: slot f of expert e goes to bases[b][e] + (number of earlier
// slots of the same block routed to e).  Earlier = smaller flat index.  Each
// round takes ROUTE_THREADS consecutive slots: a slot's rank among the slots
// of its wave routed to the same expert comes from ballots over the expert's
// bits, the waves before it add their counts (LDS, in wave order).
constexpr int ROUTE_WAVES = ROUTE_THREADS / 64;
__global__ __launch_bounds__(ROUTE_THREADS) void expert_scatter_kernel(const int32_t* __restrict__ idx, int M, int E,
                                                                       int ebits, const int32_t* __restrict__ bases,
                                                                       int32_t* __restrict__ s2f,
                                                                       int32_t* __restrict__ f2s) {
  __shared__ int s_run[MAX_E];
  __shared__ int s_wc[ROUTE_WAVES][MAX_E];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) {
    s_run[e] = bases[blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < ROUTE_WAVES; ++w) s_wc[w][e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int base = blockIdx.x * ROUTE_CHUNK;
  for (int round = 0; round < ROUTE_CHUNK / ROUTE_THREADS; ++round) {
    const int f = base + round * ROUTE_THREADS + threadIdx.x;
    const bool valid = f < M;
    const int e = valid ? idx[f] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) s_wc[wave][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int pos = s_run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wc[w][e];
      s2f[pos] = f;
      f2s[f] = pos;
    }
    __syncthreads();
    for (int ee = threadIdx.x; ee < E; ee += ROUTE_THREADS) {
      int sum = 0;
#pragma unroll
      for (int w = 0; w < ROUTE_WAVES; ++w) {
        sum += s_wc[w][ee];
        s_wc[w][ee] = 0;
      }
      s_run[ee] += sum;
    }
    __syncthreads();
  }
}

// Routing scratch of the allocation-free entry point: the per-block expert
// partials and block bases (2 * blocks * E int32), in a file-scope device
// array that every GPU the library runs on holds until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// is only a stand-in for the symbol); it takes each device's address of the
// array from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[ROUTE_SCRATCH_BYTES];

hipError_t route_scratch_ptr(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (dev_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

int resident_blocks(int per_cu) {
  constexpr int kMaxDevices = 64;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  int n = dev >= 0 ? __atomic_load_n(&cus[dev], __ATOMIC_RELAXED) : 0;
  if (n == 0) {
    if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    if (dev >= 0) __atomic_store_n(&cus[dev], n, __ATOMIC_RELAXED);
  }
  const int b = n * (per_cu > 0 ? per_cu : 1);
  return b < 8 ? 8 : b / 8 * 8;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* topk_idx, float* gate,
                        int32_t* counts, int32_t* offsets, int32_t* s2f, int32_t* f2s,
                        int32_t* ws_partials, int32_t* ws_bases, hipStream_t s) {
  const int M = T * k;
  const int nblk = route_num_blocks(M);
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  hipError_t e = k <= TOPK_SMALL
                    ? launch_kernel(topk_gate_small_kernel, dim3((T + 63) / 64), dim3(256), 0, s, logits, T, E, k,
                                    topk_idx, gate)
                    : launch_kernel(topk_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, topk_idx,
                                    gate);
  if (e == hipSuccess)
    e = launch_kernel(expert_hist_kernel, dim3(nblk), dim3(ROUTE_THREADS), 0, s, (const int32_t*)topk_idx, M, E,
                      ws_partials);
  if (e == hipSuccess)
    e = launch_kernel(expert_scan_kernel, dim3(1), dim3(1024), 0, s, (const int32_t*)ws_partials, nblk, E, ws_bases,
                      counts, offsets);
  if (e == hipSuccess)
    e = launch_kernel(expert_scatter_kernel, dim3(nblk), dim3(ROUTE_THREADS), 0, s, (const int32_t*)topk_idx, M, E,
                      ebits, (const int32_t*)ws_bases, s2f, f2s);
  return e;
}

// Tile table of the row-ragged GEMMs: tile i covers rows [row0, row0 + bm) of
// expert tile_expert[i] (clipped to the expert's end); unused tiles get -1.
// expert_tile0[e] = first tile of expert e (expert_tile0[E] = number of tiles).
// Weight-gradient work list (optional, `wg` non-null; see WgradList): the
// experts by decreasing row count, ties by index (longest-processing-time-
// first list scheduling), each split into chunks of at most WG_KC rows (an
// empty expert is one empty chunk); chunk c > 0 of an expert accumulates into
// a partial slot that the ordered reduction adds to chunk 0's result.  The
// chunks are then dealt to the 8 XCD queues (balanced load).
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                          int max_tiles, int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ tile_row0,
                                                          int32_t* __restrict__ expert_tile0, WgradList wg) {
  __shared__ int s_start[2][MAX_E + 1];
  __shared__ int s_cnt[MAX_E];
  const int e = threadIdx.x;
  int cur = 0;
  int nt = 0;
  if (e < E) {
    s_cnt[e] = offsets[e + 1] - offsets[e];
    nt = (s_cnt[e] + bm - 1) / bm;
  }
  if (e <= MAX_E) s_start[0][e] = (e < E) ? nt : 0;
  __syncthreads();
  for (int off = 1; off <= MAX_E; off <<= 1) {
    if (e <= MAX_E) {
      int val = s_start[cur][e];
      if (e >= off) val += s_start[cur][e - off];
      s_start[cur ^ 1][e] = val;
    }
    cur ^= 1;
    __syncthreads();
  }
  if (wg.order) {
    __shared__ int s_nch[MAX_E];            // chunks of the expert of each rank
    __shared__ int s_rows[MAX_E];           // rows of the expert of each rank
    if (e < E) {   // rank of e by (count desc, index asc); s_cnt is visible after the scan's barriers
      const int c = s_cnt[e];
      int rank = 0;
      for (int f = 0; f < E; ++f) rank += (s_cnt[f] > c) || (s_cnt[f] == c && f < e);
      wg.order[rank] = e;
      s_nch[rank] = c > WG_KC ? (c + WG_KC - 1) / WG_KC : 1;
      s_rows[rank] = c;
    }
    __syncthreads();
    // exclusive prefix of the chunk counts over the ranks (Hillis-Steele over
    // MAX_E entries; ranks past E count 0): cstart[r], and slot0[r] =
    // cstart[r] - r (chunks beyond each rank's first)
    __shared__ int s_cs[2][MAX_E];
    int cc = 0;
    if (e < MAX_E) s_cs[0][e] = (e < E) ? s_nch[e] : 0;
    __syncthreads();
    for (int off = 1; off < MAX_E; off <<= 1) {
      if (e < MAX_E) {
        int val = s_cs[cc][e];
        if (e >= off) val += s_cs[cc][e - off];
        s_cs[cc ^ 1][e] = val;
      }
      cc ^= 1;
      __syncthreads();
    }
    if (e < E) {
      const int excl = s_cs[cc][e] - s_nch[e];
      wg.cstart[e] = excl;
      wg.slot0[e] = excl - e;
      if (e == E - 1) wg.cstart[E] = s_cs[cc][e];
    }
    // XCD queues (cap = ceil(chunks / 8) entries each, so that the grid of
    // the weight-gradient kernels, cap chunk rounds per XCD, covers them all).
    // Even routing (no expert above twice the mean): the snake deal, filled by
    // all threads at once -- in round q the XCDs take chunks 8q .. 8q + 7, XCD
    // x chunk 8q + x in even rounds and 8q + 7 - x in odd ones.  Skewed
    // routing: the chunks in list order (decreasing rows, so longest
    // processing time first), each to the queue of least load (rows + WG_BETA
    // per chunk; ties: lowest XCD) among those holding fewer than cap.  Lanes
    // 0-7 of the first wave own one queue each; the choice is the minimum over
    // those lanes of the key load * 8 + lane (3 DPP steps: quad swaps, then
    // the half-row mirror), so all of them pick the same queue.  The experts'
    // chunk and row counts arrive 64 at a time (one LDS read per lane, then
    // readlane).
    const int n = s_cs[cc][E - 1];
    const int cap = (n + 7) / 8;
    const bool skewed = (long long)s_rows[0] * E > 2LL * offsets[E];
    if (!skewed) {
      for (int i = e; i < 8 * cap; i += blockDim.x) {
        const int x = i / cap, q = i % cap;
        const int item = 8 * q + ((q & 1) ? 7 - x : x);
        wg.xq[i] = item < n ? item : -1;
      }
    } else if (e < 64) {
      int len = 0, load = 0;
      int item = 0;
      for (int r0 = 0; r0 < E; r0 += 64) {
        const int vn = r0 + e < E ? s_nch[r0 + e] : 0;
        const int vr = r0 + e < E ? s_rows[r0 + e] : 0;
        const int nr = min(64, E - r0);
        for (int l = 0; l < nr; ++l) {
          const int nch = __builtin_amdgcn_readlane(vn, l), rows_r = __builtin_amdgcn_readlane(vr, l);
          for (int ch = 0; ch < nch; ++ch, ++item) {
            const int rows = min(rows_r - ch * WG_KC, WG_KC);
            uint32_t key = (e < 8 && len < cap) ? (uint32_t)min(load, (1 << 28) - 1) * 8u + (uint32_t)e : UINT_MAX;
            key = min(key, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)key, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
            key = min(key, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)key, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
            key = min(key, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)key, 0x141, 0xF, 0xF, false));   // row_half_mirror
            if (e == (int)(key & 7u)) {
              wg.xq[e * cap + len] = item;
              ++len;
              load += rows + WG_BETA;
            }
          }
        }
      }
      if (e < 8)
        for (int q = len; q < cap; ++q) wg.xq[e * cap + q] = -1;
    }
  }
  // s_start[cur][e] = inclusive sum; exclusive start of e = inclusive(e-1)
  const int total = s_start[cur][E - 1];
  if (e <= E) expert_tile0[e] = (e == 0) ? 0 : s_start[cur][e - 1];
  for (int t = threadIdx.x; t < max_tiles; t += 1024) {
    int ex = -1, r0 = 0;
    if (t < total) {
      int lo = 0, hi = E - 1;            // first e with inclusive(e) > t
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_start[cur][mid] > t) hi = mid; else lo = mid + 1;
      }
      ex = lo;
      const int first = (lo == 0) ? 0 : s_start[cur][lo - 1];
      r0 = offsets[lo] + (t - first) * bm;
    }
    tile_expert[t] = ex;
    tile_row0[t] = r0;
  }
}

hipError_t launch_tile_table(const int32_t* offsets, int E, int bm, int max_tiles, int32_t* tile_expert,
                             int32_t* tile_row0, int32_t* expert_tile0, WgradList wg, hipStream_t s) {
  return launch_kernel(tile_table_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bm, max_tiles, tile_expert,
                       tile_row0, expert_tile0, wg);
}

}  // namespace moe
