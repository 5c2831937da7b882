// Ragged grouped GEMMs of the MoE backward pass on MXFP8 operands (gfx950,
// v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3FN codes and E8M0 block
// scales), fp32 accumulation, with the same fused epilogues as the bf16 path.
//
// fp8_bwd mode: the forward stays in bf16 and every backward GEMM reads both
// operands as MXFP8, quantised in blocks of 32 along that GEMM's K, the token
// blocks group-aware per expert (Prime Mega MoE news page, "How does the
// fused kernel work?": an fp8_bwd mode, BF16 forward and FP8 backward; TE
// dropless-MoE page, "03 Specialised optimisations": group-aware MXFP8
// quantisation with MXFP8 grouped GEMM).
//
// mxfp8 mode (the same page's BF16/MXFP8 precisions): the forward GEMMs too.
//
// Every kernel computes C[m][n] = sum_k A[m][k] B[n][k] over one BM x BN
// tile, both operands stored K-contiguous (codes [rows][K], scales
// [rows][K/32]):
//   GEMM W13 + SwiGLU (KIND_FWD1): A = x[tok(r)] (gathered), B = W13[e] rows; K = H
//   GEMM W2      (KIND_FWD2):  A = A rows,               B = W2[e] rows;  K = I
//   dgrad of W2   (KIND_DGRAD2): A = dY[tok(r)] (gathered), B = W2[e]^T;  K = H
//   dgrad of W13  (KIND_DGRAD1): A = dG13 rows,            B = W13[e]^T; K = 2I
//   wgrad of W2   (KIND_WGRAD2): A = dY^T, B = (gate A)^T;   K = tokens of e
//   wgrad of W13  (KIND_WGRAD1): A = dG13^T, B = x^T;        K = tokens of e
// One K tile = 128 codes = one scaled MFMA step.  Lane l of a fragment holds
// 32 codes of row l%16: K bytes 16g .. 16g+15 and 64+16g .. 64+16g+15 of the
// tile (g = l/16), and the scale byte of K block g (bytes 32g .. 32g+31) of
// that row (lane layout checked against a CPU product on the device).  The
// MFMA's first operand is the B tile, so lane l holds D[n = 4*(l/16) + v][m =
// l%16], the layout the shared epilogues expect.  The epilogue of the dgrad
// of W2 reads the fp32 G13 saved in these modes and quantises dG13 and
// gate*A from fp32 registers straight into the MXFP8 operands of the three
// GEMMs that follow (row blocks for the dgrad of W13, token blocks for both
// weight gradients).
//
// LDS stage: A codes [BM][128], B codes [BN][128] (16-byte chunks XOR-swizzled
// by row & 7, conflict-free two-chunk reads), then A scales [BM][4] and B
// scales [BN][4].  Codes arrive by 16-byte and scales by 4-byte buffer-to-LDS
// DMA; offsets past a buffer's end read zeros.  Two main loops: as in the
// bf16 kernels (STAGES tiles in flight, fragments read into registers between
// two barriers, then the freed stage is refilled while the MFMAs run), or a
// software pipeline over the wave's 16-row blocks of A with one barrier per K
// tile (see the PIPE branch).
#include "gemm_common.h"

namespace moe {
namespace {

using gg::TileCfg;
using gg::NXCD;
using gg::OOB;
using gg::make_rsrc;
using gg::dma16;
using gg::dma4;
using gg::vm_wait;
using gg::u32x4_t;

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

constexpr int KT = MX_KTILE;          // K per tile (bytes per row of a code tile)
constexpr int ROWB = KT;              // bytes per LDS code row
static_assert(KT == 128, "one scaled MFMA step per K tile");

__device__ __forceinline__ int chunk_off(int row, int chunk) {   // byte offset in a code tile
  return row * ROWB + ((chunk ^ (row & 7)) << 4);
}

// Fragment of 16 rows from row0: lane l reads logical chunks g and 4 + g (g = l/16) of row row0 + l%16.
__device__ __forceinline__ i32x8_t frag_codes(const uint8_t* tile, int row0, int lane) {
  const int row = row0 + (lane & 15), g = lane >> 4;
  const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(tile + chunk_off(row, g));
  const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(tile + chunk_off(row, g + 4));
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ __forceinline__ int frag_scale(const uint8_t* stile, int row0, int lane) {
  return stile[(row0 + (lane & 15)) * 4 + (lane >> 4)];
}

template <int KIND> struct MxKind {
  static constexpr bool ragged_rows = (KIND != KIND_WGRAD2 && KIND != KIND_WGRAD1);
};

template <int KIND, class C>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void gemm_mx8_kernel(LayerArgs a, Mx8Args q, int n_tiles, int tiles_total, int nvb) {
  constexpr int BM = C::BM, BN = C::BN, NTHR = C::NTHR, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int NW = C::NW, S = C::STAGES;
  constexpr int DA = BM * ROWB / 1024 / NW, DB = BN * ROWB / 1024 / NW;   // 1 KiB code DMAs per wave
  constexpr int SA = BM * 4 / 256, SB = BN * 4 / 256;                     // 256-byte scale DMAs per tile
  // scale DMAs per wave; when they do not split evenly over the waves, the
  // spare ones read zeros (an offset past the buffer) into a pad block, so
  // that every wave issues the same number of DMA instructions per tile
  constexpr int DS = (SA + SB + NW - 1) / NW;
  static_assert(DA * NW * 1024 == BM * ROWB && DB * NW * 1024 == BN * ROWB, "code tiles split into 1 KiB DMAs");
  static_assert(SA * 256 == BM * 4 && SB * 256 == BN * 4, "scale rows split into 256-byte DMAs");
  constexpr int A_CODES = 0, B_CODES = BM * ROWB, A_SC = (BM + BN) * ROWB, B_SC = A_SC + BM * 4;
  constexpr int PAD = B_SC + BN * 4;                                      // pad block of the spare scale DMAs
  constexpr int STAGE = (BM + BN) * (ROWB + 4) + (DS * NW > SA + SB ? 256 : 0);
  constexpr int PER_WAVE = DA + DB + DS;   // DMA instructions per wave per K tile
  // operand stages, or the staging of the dgrad-of-W2 epilogue when larger
  constexpr int EPI_LDS = KIND == KIND_DGRAD2 ? gg::dgrad2_mx8_lds_bytes<C>() : 0;
  constexpr int LDS_BYTES = S * STAGE > EPI_LDS ? S * STAGE : EPI_LDS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];


  // The block takes the virtual blocks vb = blockIdx.x, blockIdx.x + gridDim.x,
  // ... below nvb (one when the grid covers them all; a persistent block
  // otherwise)
  auto tile_body = [&](const int vb) __attribute__((always_inline)) {
  // the thread index passes through an empty asm statement, so that nothing
  // derived from it is hoisted out of a persistent block's tile loop (that
  // would keep per-lane addresses live across the epilogue)
  int tid = threadIdx.x;
  if constexpr (C::PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int H = a.H, I = a.I, k = a.k;
  // ---------------- tile decode (row kinds: XCD-contiguous renumbering of the
  // tile table; weight gradients: experts by decreasing size, see decode_wgrad_tile)
  int e, m0, mlim, n0, nk, kp0 = 0;
  float* wout = nullptr;   // weight gradients: dW[e], or the chunk's partial slot
  bool wacc = false;       //   dW[e] adds the caller's value (accumulate-into)
  if constexpr (MxKind<KIND>::ragged_rows) {
    const int per_xcd = nvb / NXCD;
    const int L = (vb % NXCD) * per_xcd + vb / NXCD;
    if (L >= tiles_total) return;
    gg::RowTile rt;
    if (!gg::decode_row_tile(a, L, n_tiles, C::GROUP, rt)) return;
    e = rt.e;
    m0 = rt.m0;
    mlim = rt.mlim;
    n0 = rt.nt * (KIND == KIND_FWD1 ? BN / 2 : BN);
    nk = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2 ? H : KIND == KIND_FWD2 ? I : 2 * I) / KT;
  } else {
    const int per_e = n_tiles * (((KIND == KIND_WGRAD2 ? H : 2 * I) + BM - 1) / BM);
    int t, r0, r1, slot;
    if (!decode_wgrad_tile(a, vb, per_e, e, r0, r1, slot, t)) return;
    m0 = (t / n_tiles) * BM;
    n0 = (t % n_tiles) * BN;
    kp0 = q.pad_off[e] + r0;              // chunks start on K-tile boundaries of the padded rows
    nk = (r1 - r0 + KT - 1) / KT;
    wout = gg::wgrad_out<KIND>(a, e, slot);
    wacc = a.wgrad_acc && slot < 0;
    mlim = (KIND == KIND_WGRAD2) ? H : 2 * I;
  }
  const int nlim = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2 || KIND == KIND_WGRAD2) ? I : H;

  // ---------------- operands ----------------
  // codes / scales buffers, row length in bytes (K) of each operand
  const uint8_t *ca, *sa_, *cb, *sb_;
  int lda, ldb, arows, brows;
  if constexpr (KIND == KIND_FWD1) {           // x rows (gathered) x W13[e] rows, K = H
    ca = q.qx; sa_ = q.sx; lda = H; arows = a.T;
    cb = q.qw13 + (size_t)e * 2 * I * H; sb_ = q.sw13 + (size_t)e * 2 * I * (H / 32); ldb = H; brows = 2 * I;
  } else if constexpr (KIND == KIND_FWD2) {    // A rows x W2[e] rows, K = I
    ca = q.qa; sa_ = q.sa; lda = I; arows = a.M;
    cb = q.qw2 + (size_t)e * H * I; sb_ = q.sw2 + (size_t)e * H * (I / 32); ldb = I; brows = H;
  } else if constexpr (KIND == KIND_DGRAD2) {
    ca = q.qdy; sa_ = q.sdy; lda = H; arows = a.T;
    cb = q.qw2t + (size_t)e * I * H; sb_ = q.sw2t + (size_t)e * I * (H / 32); ldb = H; brows = I;
  } else if constexpr (KIND == KIND_DGRAD1) {
    ca = q.qdg; sa_ = q.sdg; lda = 2 * I; arows = a.M;
    cb = q.qw13t + (size_t)e * H * 2 * I; sb_ = q.sw13t + (size_t)e * H * (2 * I / 32); ldb = 2 * I; brows = H;
  } else if constexpr (KIND == KIND_WGRAD2) {
    ca = q.qdyt; sa_ = q.sdyt; lda = q.Mp; arows = H;
    cb = q.qagt; sb_ = q.sagt; ldb = q.Mp; brows = I;
  } else {
    ca = q.qdgt; sa_ = q.sdgt; lda = q.Mp; arows = 2 * I;
    cb = q.qxt; sb_ = q.sxt; ldb = q.Mp; brows = H;
  }
  const __amdgpu_buffer_rsrc_t rca = make_rsrc(ca, (uint32_t)((size_t)arows * lda));
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa_, (uint32_t)((size_t)arows * (lda / 32)));
  const __amdgpu_buffer_rsrc_t rcb = make_rsrc(cb, (uint32_t)((size_t)brows * ldb));
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sb_, (uint32_t)((size_t)brows * (ldb / 32)));

  // source row (of the operand's buffer) of tile row rl
  auto a_src_row = [&](int rl) -> uint32_t {
    if constexpr (KIND == KIND_DGRAD2 || KIND == KIND_FWD1) return (uint32_t)(a.s2f[min(m0 + rl, mlim - 1)] / k);
    else return (uint32_t)min(m0 + rl, mlim - 1);
  };
  auto b_src_row = [&](int nl) -> uint32_t {
    if constexpr (KIND == KIND_FWD1) {         // tile rows [0, BN/2) are W1 rows, the rest the matching W3 rows
      const int c = min(n0 + (nl & (BN / 2 - 1)), I - 1);
      return (uint32_t)((nl < BN / 2) ? c : I + c);
    } else {
      return (uint32_t)min(n0 + nl, nlim - 1);
    }
  };
  // LDS row of the j-th 16-row MFMA block of this wave's B sub-tile (the
  // SwiGLU kind pairs each W1 block with its W3 block)
  auto brow = [&](int j) -> int {
    if constexpr (KIND == KIND_FWD1)
      return (j < FN / 2) ? wn * (WN / 2) + 16 * j : BN / 2 + wn * (WN / 2) + 16 * (j - FN / 2);
    else
      return wn * WN + 16 * j;
  };

  // DMA instruction i of wave w fills 1 KiB block ci = i*NW + w of a code
  // tile: 8 rows of 128 bytes; lane l writes physical chunk l%8 of row
  // 8 ci + l/8, which holds logical chunk (l%8) ^ (row & 7).
  const int w_uni = __builtin_amdgcn_readfirstlane(wave);
  uint32_t oa[DA], ob[DB];
#pragma unroll
  for (int i = 0; i < DA; ++i) {
    const int rl = 8 * (i * NW + w_uni) + lane / 8;
    oa[i] = a_src_row(rl) * (uint32_t)lda + (uint32_t)kp0 + (uint32_t)(((lane & 7) ^ (rl & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int nl = 8 * (i * NW + w_uni) + lane / 8;
    ob[i] = b_src_row(nl) * (uint32_t)ldb + (uint32_t)kp0 + (uint32_t)(((lane & 7) ^ (nl & 7)) << 4);
  }
  // scale DMA j (global index w + NW*j over SA + SB): 64 rows x 4 bytes
  uint32_t os[DS];
  bool os_b[DS];
#pragma unroll
  for (int j = 0; j < DS; ++j) {
    const int g = w_uni + NW * j;
    if (g < SA) {
      os[j] = a_src_row(64 * g + lane) * (uint32_t)(lda / 32) + (uint32_t)(kp0 / 32);
      os_b[j] = false;
    } else if (g < SA + SB) {
      os[j] = b_src_row(64 * (g - SA) + lane) * (uint32_t)(ldb / 32) + (uint32_t)(kp0 / 32);
      os_b[j] = true;
    } else {
      os[j] = OOB;                       // spare: zeros into the pad block
      os_b[j] = true;
    }
  }
  // LDS byte offset (in a stage) of scale DMA j of this wave
  auto sc_dst = [&](int j) __attribute__((always_inline)) -> uint32_t {
    const int g = w_uni + NW * j;
    return g < SA ? (uint32_t)(A_SC + g * 256) : g < SA + SB ? (uint32_t)(B_SC + (g - SA) * 256) : (uint32_t)PAD;
  };

  const uint32_t lds0 = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)smem;
  auto issue_tile = [&](int kt, int st) __attribute__((always_inline)) {
    const bool live = kt < nk;
    const uint32_t sbase = lds0 + (uint32_t)(st * STAGE);
    const uint32_t kb = (uint32_t)kt * KT;
#pragma unroll
    for (int i = 0; i < DA; ++i)
      dma16(rca, live ? oa[i] + kb : OOB, __builtin_amdgcn_readfirstlane(sbase + A_CODES + (i * NW + w_uni) * 1024));
#pragma unroll
    for (int i = 0; i < DB; ++i)
      dma16(rcb, live ? ob[i] + kb : OOB, __builtin_amdgcn_readfirstlane(sbase + B_CODES + (i * NW + w_uni) * 1024));
#pragma unroll
    for (int j = 0; j < DS; ++j) {
      const uint32_t off = (live && os[j] != OOB) ? os[j] + (uint32_t)kt * 4 : OOB;
      dma4(os_b[j] ? rsb : rsa, off, __builtin_amdgcn_readfirstlane(sbase + sc_dst(j)));
    }
  };

  // DMA instruction q (< PER_WAVE) of this wave for K tile kt into stage st:
  // A codes, then B codes, then scales
  auto issue_q = [&](int kt, int st, int q) __attribute__((always_inline)) {
    const bool live = kt < nk;
    const uint32_t sbase = lds0 + (uint32_t)(st * STAGE);
    const uint32_t kb = (uint32_t)kt * KT;
    if (q < DA) {
      dma16(rca, live ? oa[q] + kb : OOB, __builtin_amdgcn_readfirstlane(sbase + A_CODES + (q * NW + w_uni) * 1024));
    } else if (q < DA + DB) {
      const int i = q - DA;
      dma16(rcb, live ? ob[i] + kb : OOB, __builtin_amdgcn_readfirstlane(sbase + B_CODES + (i * NW + w_uni) * 1024));
    } else {
      const int j = q - DA - DB;
      const uint32_t off = (live && os[j] != OOB) ? os[j] + (uint32_t)kt * 4 : OOB;
      dma4(os_b[j] ? rsb : rsa, off, __builtin_amdgcn_readfirstlane(sbase + sc_dst(j)));
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // a wave whose rows all lie past the expert's end (the ragged last tile)
  // keeps its share of the DMA and the barriers and skips its fragment reads
  // and MFMAs: its accumulators stay zero, which the epilogues read as the
  // zero rows of the padded tile
  const bool idle = MxKind<KIND>::ragged_rows &&
                    __builtin_amdgcn_readfirstlane((int)(m0 + wm * WM >= mlim)) != 0;
  if constexpr (C::PIPE) {
    // Software pipeline over the wave's 16-row blocks of A (one K tile = one
    // scaled-MFMA step).  All FN fragments of B stay in registers for the
    // tile; the A fragment of row block i is read two blocks ahead (four
    // rotating registers).  One barrier per K tile, at the start of row block
    // FM-2: every read of this tile's stage is then complete and the DMA of
    // tile kt+1 has landed, so the stage receives tile kt+S over the last two
    // row blocks, whose MFMAs also overlap the reads of the next tile: its
    // first two A fragments, and B fragment j right after its last use here.
    static_assert(FM % 4 == 0 || FM == 2, "rotating A registers");
    constexpr int NA = FM >= 4 ? 4 : 2;
    i32x8_t ar[NA], br[FN];
    int sa[NA], sb[FN];
    auto read_a = [&](int st, int i, int slot) __attribute__((always_inline)) {
      const uint8_t* base = smem + st * STAGE;
      ar[slot] = frag_codes(base + A_CODES, wm * WM + 16 * i, lane);
      sa[slot] = frag_scale(base + A_SC, wm * WM + 16 * i, lane);
    };
    auto read_b = [&](int st, int j) __attribute__((always_inline)) {
      const uint8_t* base = smem + st * STAGE;
      br[j] = frag_codes(base + B_CODES, brow(j), lane);
      sb[j] = frag_scale(base + B_SC, brow(j), lane);
    };
    auto lds_wait_all = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0xC07F); };
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int q = 0; q < PER_WAVE; ++q) issue_q(st, st, q);
    vm_wait<(S - 1) * PER_WAVE>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int st_c = 0;
    if (idle) {
      for (int kt = 0; kt < nk; ++kt) {
        vm_wait<(S - 2) * PER_WAVE>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) issue_q(kt + S, st_c, q);
        st_c = (st_c + 1 == S) ? 0 : st_c + 1;
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) read_b(0, j);
      read_a(0, 0, 0);
      read_a(0, 1, 1);
      for (int kt = 0; kt < nk; ++kt) {
        const int st_n = (st_c + 1 == S) ? 0 : st_c + 1;
        constexpr int NB_LAST = 2 * FN;                            // MFMAs of the last two row blocks
        constexpr int SP = NB_LAST / PER_WAVE > 0 ? NB_LAST / PER_WAVE : 1;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int slot = i % NA;
          if (i == FM - 2) {                                       // publish tile kt+1, free this stage
            lds_wait_all();
            vm_wait<(S - 2) * PER_WAVE>();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
          }
          // the A fragment two row blocks ahead (of the next tile past FM-2)
          if (i + 2 < FM) read_a(st_c, i + 2, (i + 2) % NA);
          else read_a(st_n, i + 2 - FM, (i + 2) % NA);
          __builtin_amdgcn_sched_barrier(0);                        // issued before this row's MFMAs
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(br[j], ar[slot], acc[i][j], 0, 0, 0, sb[j],
                                                                         0, sa[slot]);
            if (i == FM - 1) read_b(st_n, j);                      // B fragment j of the next tile
            if (i >= FM - 2) {
              const int idx = (i - (FM - 2)) * FN + j;
              if (idx % SP == SP - 1 && idx / SP < PER_WAVE) {
                issue_q(kt + S, st_c, idx / SP);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
        }
#pragma unroll
        for (int q = NB_LAST / SP; q < PER_WAVE; ++q) issue_q(kt + S, st_c, q);
        st_c = st_n;
      }
    }
  } else {

  i32x8_t af[FM], bfr[FN];
  int as[FM], bs[FN];
  auto load_frags = [&](int st) __attribute__((always_inline)) {
    const uint8_t* base = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      af[i] = frag_codes(base + A_CODES, wm * WM + 16 * i, lane);
      as[i] = frag_scale(base + A_SC, wm * WM + 16 * i, lane);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bfr[j] = frag_codes(base + B_CODES, brow(j), lane);
      bs[j] = frag_scale(base + B_SC, brow(j), lane);
    }
  };
  auto mfmas = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0, 0, bs[j], 0,
                                                                     as[i]);
  };

  // ---------------- main loop ----------------
#pragma unroll
  for (int st = 0; st < S; ++st) issue_tile(st, st);
  int st_c = 0;
  if (idle) {
    for (int kt = 0; kt < nk; ++kt) {
      vm_wait<(S - 1) * PER_WAVE>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_tile(kt + S, st_c);
      st_c = (st_c + 1 == S) ? 0 : st_c + 1;
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      vm_wait<(S - 1) * PER_WAVE>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      load_frags(st_c);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_tile(kt + S, st_c);
      mfmas();
      st_c = (st_c + 1 == S) ? 0 : st_c + 1;
    }
  }
  }
  vm_wait<0>();      // no DMA may land while the epilogue reuses LDS
  __syncthreads();

  if constexpr (KIND == KIND_DGRAD2)
    gg::dgrad2_epilogue_mx8<C, LDS_BYTES>(a, q, acc, smem, tid, lane, wm, wn, e, m0, mlim, n0);
  else
    gg::gemm_epilogue<KIND, C, true>(a, acc, smem, tid, lane, wm, wn, e, m0, mlim, n0, nlim, wout, wacc);
  };
  if constexpr (C::PERSIST) {
    for (int vb = blockIdx.x; vb < nvb; vb += gridDim.x) {
      tile_body(vb);
      __syncthreads();   // every wave is done with the LDS before the next tile's DMA lands
    }
  } else {
    tile_body(blockIdx.x);
  }
}

// Tile shapes (BM x BN, waves WGM x WGN, waves per SIMD, LDS stages, tile
// group divisor, main loop).  The BK of TileCfg is 64: its bf16 byte count
// per row (128) is the MXFP8 K tile.  Forward kinds: 256 x 256 tiles, 8
// waves, tile groups of 8 blocks (GEMM W13 13 % and GEMM W2 5 % faster than
// 128 x 128: half the operand bytes per flop).  Weight gradients: 256 x 256
// tiles on 4 waves of 128 x 128 with the software-pipelined loop (one wave
// per SIMD, 4-5 % faster than 8 waves with the two-barrier loop).  The dgrad
// kinds stay at 128 x 128 (the dgrad-of-W2 epilogue writes one padded
// 128-token K tile of the weight-gradient operands per tile; 128 x 256 with
// 4 or 8 waves measured slower).
#ifndef MOE_MX8_CFG_ROW
#define MOE_MX8_CFG_ROW 128, 128, 2, 2, 2, 2, 64
#endif
#ifndef MOE_MX8_CFG_WGRAD
#define MOE_MX8_CFG_WGRAD 256, 256, 2, 2, 1, 2, 64, 1, 1
#endif
#ifndef MOE_MX8_CFG_ROW_FWD
#define MOE_MX8_CFG_ROW_FWD 256, 256, 2, 4, 2, 2, 64, 4
#endif
using CfgRowF = TileCfg<MOE_MX8_CFG_ROW_FWD>;   // forward kinds (their own tile table)
using CfgRow = TileCfg<MOE_MX8_CFG_ROW>;
using CfgW = TileCfg<MOE_MX8_CFG_WGRAD>;

template <int KIND, class C>
hipError_t launch_kind(const LayerArgs& a, const Mx8Args& q, hipStream_t s) {
  int n_tiles, tiles;
  if constexpr (MxKind<KIND>::ragged_rows) {
    const int ncols = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2) ? a.I : a.H;
    const int bn = (KIND == KIND_FWD1) ? C::BN / 2 : C::BN;
    n_tiles = (ncols + bn - 1) / bn;
    tiles = n_tiles * max_row_tiles(a.M, a.E, C::BM);
  } else {
    const int mdim = (KIND == KIND_WGRAD2) ? a.H : 2 * a.I;
    const int ndim = (KIND == KIND_WGRAD2) ? a.I : a.H;
    n_tiles = (ndim + C::BN - 1) / C::BN;
    tiles = a.E * n_tiles * ((mdim + C::BM - 1) / C::BM);
  }
  const int nvb = MxKind<KIND>::ragged_rows ? (tiles + NXCD - 1) / NXCD * NXCD
                                            : wgrad_grid(wgrad_max_chunks(a.M, a.E), tiles / a.E);
  const int grid = C::PERSIST ? min(nvb, resident_blocks(C::WPE * 4 / C::NW)) : nvb;
  return launch_kernel((gemm_mx8_kernel<KIND, C>), dim3(grid), dim3(C::NTHR), 0, s, a, q, n_tiles, tiles, nvb);
}

}  // namespace

int mx8_fwd_row_tile_m() { return CfgRowF::BM; }
int mx8_row_tile_m() { return CfgRow::BM; }
int mx8_dgrad2_tile_n() { return CfgRow::BN; }

hipError_t launch_gemm_mx8(GemmKind kind, const LayerArgs& a, const Mx8Args& q, hipStream_t s) {
  switch (kind) {
    case KIND_FWD1: return launch_kind<KIND_FWD1, CfgRowF>(a, q, s);
    case KIND_FWD2: return launch_kind<KIND_FWD2, CfgRowF>(a, q, s);
    case KIND_DGRAD2: return launch_kind<KIND_DGRAD2, CfgRow>(a, q, s);
    case KIND_DGRAD1: return launch_kind<KIND_DGRAD1, CfgRow>(a, q, s);
    case KIND_WGRAD2: return launch_kind<KIND_WGRAD2, CfgW>(a, q, s);
    case KIND_WGRAD1: return launch_kind<KIND_WGRAD1, CfgW>(a, q, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
