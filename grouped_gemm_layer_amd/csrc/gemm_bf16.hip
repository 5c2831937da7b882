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
// Every kernel computes C[m][n] = sum_k A[m][k] B[n][k] over one BM x BN tile:
//   row-ragged kinds (forward, dgrad): m = expert-sorted token rows of one
//     expert (tile table), n = output features, K = H, I or 2I;
//   wgrad kinds: m, n = weight-gradient rows/cols of one expert, K = that
//     expert's token rows, ragged and zero-padded.
// Operands come in two global layouts:
//   KC: element (row, k) at row_ptr(row)[k]   (K contiguous)
//   KO: element (row, k) at krow_ptr(k)[row]  (rows contiguous)
// KC tiles are stored in LDS as [row][64 k] with 16-byte chunks XOR-swizzled by
// row and read with ds_read_b128; KO tiles keep their global layout in LDS,
// [64 k][R rows] with 32-byte granules XOR-swizzled by k, and are read with two
// ds_read_b64_tr_b16 (gfx950 LDS transpose reads: within each 16-lane group,
// lane d receives element d%4 of the 8-byte reads of lanes 4j + d/4, j = 0..3).
// Either way an MFMA operand register holds 8 consecutive k of one row, so the
// layouts mix freely.
//
// The MFMA's first operand is the B tile (rows n) and its second the A tile
// (rows m): lane l holds D[n = 4*(l/16) + v][m = l%16], i.e. four consecutive
// output features of one row, stored as one 8- or 16-byte write.
//
// Operands travel by buffer-to-LDS DMA (16 bytes per lane, 1 KiB per
// instruction): an offset past the buffer's end stores zeros, which pads the
// ragged K tail of the wgrad GEMMs without branches.  Pipeline: STAGES LDS
// stages; per K tile every wave reads its MFMA fragments into registers
// between two barriers, then the DMA instructions of the tile STAGES ahead are
// issued one by one between its MFMAs.  The token offsets of the gathered
// wgrad rows come from an LDS table refilled every 2048 rows.
// Blocks are renumbered so that each XCD (8 per chip, blocks dealt
// round-robin) receives a contiguous range of the expert-major tile order and
// its L2 serves the shared weight and token panels.
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int TOKTAB = 2048;                 // gathered K rows per LDS token table
using gg::TileCfg;
using gg::NXCD;
using gg::OOB;
using gg::make_rsrc;
using gg::dma16;
using gg::vm_wait;
using gg::u32x4_t;

// ---- LDS layouts (element offsets) ----
// KC: [row][BK], 16-byte chunk c of row r stored at chunk c ^ swz(r).  With
// 128-byte rows, swz = r & 7 makes the fragment reads (16 rows x one chunk per
// 16 lanes) conflict-free on gfx950 (measured: ~190 B/clk/CU against ~113 for
// swz = (r ^ r>>3) & 7, which conflicts two-way).
template <int BK>
__device__ __forceinline__ int kc_swz(int row) {
  if constexpr (BK == 64) return row & 7;
  else return ((row >> 1) ^ (row >> 2)) & 3;
}
template <int BK>
__device__ __forceinline__ int kc_off(int row, int chunk) {
  return row * BK + ((chunk ^ kc_swz<BK>(row)) << 3);
}
// KO: [BK k][R], 32-byte granule g of k-row k stored at granule g ^ f(k);
// f spreads the 16 k-rows one transpose read touches over distinct granules.
template <int R>
__device__ __forceinline__ int ko_f(int k) {
  if constexpr (R >= 256) return (k & 3) | (((k >> 3) & 3) << 2);
  else if constexpr (R == 128) return (k & 3) | (((k >> 3) & 1) << 2);
  else return k & 3;
}
template <int R>
__device__ __forceinline__ int ko_off(int k, int col) {
  return k * R + ((((col >> 4) ^ ko_f<R>(k)) << 4) | (col & 15));
}

// MFMA operand fragment: 16 rows starting at `row0`, k = 32*ks + 8*(lane/16) + 0..7
template <int BK>
__device__ __forceinline__ bf16x8_t frag_kc(const bf16_t* lds, int row0, int ks, int lane) {
  return *reinterpret_cast<const bf16x8_t*>(lds + kc_off<BK>(row0 + (lane & 15), ks * 4 + (lane >> 4)));
}
template <int R>
__device__ __forceinline__ bf16x8_t frag_ko(const bf16_t* lds, int row0, int ks, int lane) {
  const int s = lane & 15;
  const int k = ks * 32 + 8 * (lane >> 4) + (s >> 2);
  const int col = row0 + 4 * (s & 3);
  const bf16_t* p0 = lds + ko_off<R>(k, col);
  const bf16_t* p1 = lds + ko_off<R>(k + 4, col);
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p0));
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- per-kind operand description ----
template <int KIND> struct Kind;
template <> struct Kind<KIND_FWD1> {   // A = x[tok(r)] (KC), B = W13 rows, G1/G3 paired (KC); K = H
  static constexpr bool ragged_rows = true, a_ko = false, b_ko = false, a_gk = false, b_gk = false;
};
template <> struct Kind<KIND_FWD2> {   // A = A rows (KC), B = W2 rows (KC); K = I
  static constexpr bool ragged_rows = true, a_ko = false, b_ko = false, a_gk = false, b_gk = false;
};
template <> struct Kind<KIND_DGRAD2> { // A = dY[tok(r)] (KC), B[n=i][k=h] = W2[h][i] (KO); K = H
  static constexpr bool ragged_rows = true, a_ko = false, b_ko = true, a_gk = false, b_gk = false;
};
template <> struct Kind<KIND_DGRAD1> { // A = dG13 rows (KC), B[n=h][k=j] = W13[j][h] (KO); K = 2I
  static constexpr bool ragged_rows = true, a_ko = false, b_ko = true, a_gk = false, b_gk = false;
};
template <> struct Kind<KIND_WGRAD2> { // A[m=h][k=r] = dY[tok(r)][h] (KO, gathered), B[n=i][k=r] = Ag[r][i] (KO)
  static constexpr bool ragged_rows = false, a_ko = true, b_ko = true, a_gk = true, b_gk = false;
};
template <> struct Kind<KIND_WGRAD1> { // A[m=j][k=r] = dG13[r][j] (KO), B[n=h][k=r] = x[tok(r)][h] (KO, gathered)
  static constexpr bool ragged_rows = false, a_ko = true, b_ko = true, a_gk = false, b_gk = true;
};


template <int KIND, class C>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void gemm_bf16_kernel(LayerArgs a, int n_tiles, int tiles_total, int nvb) {
  using K_ = Kind<KIND>;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NTHR = C::NTHR, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int DA = C::DA, DB = C::DB, NW = C::NW;
  constexpr bool gathered_k = K_::a_gk || K_::b_gk;

  constexpr int S = C::STAGES, STAGE = (BM + BN) * BK;   // elements per stage: A tile then B tile
  __shared__ __attribute__((aligned(1024))) bf16_t smem[S * STAGE];
  __shared__ uint32_t s_tok[gathered_k ? TOKTAB : 1];   // element offset of each gathered row


  // The block takes the virtual blocks vb = blockIdx.x, blockIdx.x + gridDim.x,
  // ... below nvb (one when the grid covers them all; a persistent block
  // otherwise, which starts its next tile while the stores of the last one
  // drain)
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
  int e, m0, mlim, n0, klo = 0, khi = 0, nk;
  float* wout = nullptr;   // weight gradients: dW[e], or the chunk's partial slot
  bool wacc = false;       //   dW[e] adds the caller's value (accumulate-into)
  if constexpr (K_::ragged_rows) {
    const int per_xcd = nvb / NXCD;
    const int L = (vb % NXCD) * per_xcd + vb / NXCD;
    if (L >= tiles_total) return;
    gg::RowTile rt;
    if (!gg::decode_row_tile(a, L, n_tiles, C::GROUP, rt)) return;
    e = rt.e;
    m0 = rt.m0;
    mlim = rt.mlim;
    const int nt = rt.nt;
    n0 = nt * (KIND == KIND_FWD1 ? BN / 2 : BN);
    const int Kd = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2) ? H : (KIND == KIND_FWD2 ? I : 2 * I);
    nk = Kd / BK;
  } else {
    const int per_e = n_tiles * (((KIND == KIND_WGRAD2 ? H : 2 * I) + BM - 1) / BM);
    int t, r0, r1, slot;
    if (!decode_wgrad_tile(a, vb, per_e, e, r0, r1, slot, t)) return;
    m0 = (t / n_tiles) * BM;
    n0 = (t % n_tiles) * BN;
    klo = a.offsets[e] + r0;
    khi = a.offsets[e] + r1;
    nk = (khi - klo + BK - 1) / BK;
    wout = gg::wgrad_out<KIND>(a, e, slot);
    wacc = a.wgrad_acc && slot < 0;
    mlim = (KIND == KIND_WGRAD2) ? H : 2 * I;
  }
  const int nlim = (KIND == KIND_FWD1 || KIND == KIND_DGRAD2 || KIND == KIND_WGRAD2) ? I : H;

  // ---------------- buffer resources ----------------
  const size_t M = (size_t)a.M;
  __amdgpu_buffer_rsrc_t ra_src, rb_src;
  if constexpr (KIND == KIND_FWD1) {
    ra_src = make_rsrc(a.x, (uint32_t)((size_t)a.T * H * 2));
    rb_src = make_rsrc(static_cast<const bf16_t*>(a.w13) + (size_t)e * 2 * I * H, (uint32_t)((size_t)2 * I * H * 2));
  } else if constexpr (KIND == KIND_FWD2) {
    ra_src = make_rsrc(a.A, (uint32_t)(M * I * 2));
    rb_src = make_rsrc(static_cast<const bf16_t*>(a.w2) + (size_t)e * H * I, (uint32_t)((size_t)H * I * 2));
  } else if constexpr (KIND == KIND_DGRAD2) {
    ra_src = make_rsrc(a.dy, (uint32_t)((size_t)a.T * H * 2));
    rb_src = make_rsrc(static_cast<const bf16_t*>(a.w2) + (size_t)e * H * I, (uint32_t)((size_t)H * I * 2));
  } else if constexpr (KIND == KIND_DGRAD1) {
    ra_src = make_rsrc(a.dG13, (uint32_t)(M * 2 * I * 2));
    rb_src = make_rsrc(static_cast<const bf16_t*>(a.w13) + (size_t)e * 2 * I * H, (uint32_t)((size_t)2 * I * H * 2));
  } else if constexpr (KIND == KIND_WGRAD2) {
    ra_src = make_rsrc(a.dy, (uint32_t)((size_t)a.T * H * 2));
    rb_src = make_rsrc(a.Ag, (uint32_t)(M * I * 2));
  } else {
    ra_src = make_rsrc(a.dG13, (uint32_t)(M * 2 * I * 2));
    rb_src = make_rsrc(a.x, (uint32_t)((size_t)a.T * H * 2));
  }

  // ---------------- DMA addressing ----------------
  // DMA instruction i of wave w fills LDS row-block ci = i*NW + w (1 KiB) of
  // an operand tile; lane l writes its 16 bytes at byte 1024*ci + 16*l.
  //   KC tile [row][BK]: row = (1024/(2 BK))*ci + l/(BK/8), physical chunk
  //     l%(BK/8) holds logical chunk (l%(BK/8)) ^ swz(row), i.e. global
  //     columns 8*logical .. +7 of the K tile.
  //   KO tile [64 k][R]: k = (1024*ci + 16*l) / (2R); the 32-byte granule at
  //     physical position g holds logical granule g ^ f(k).
  const int w_uni = __builtin_amdgcn_readfirstlane(wave);
  // KC source offset of this lane's 16 bytes in 1 KiB block ci of the A / B tile
  auto a_kc_off = [&](int ci) __attribute__((always_inline)) -> uint32_t {
    const int rl = (512 / BK) * ci + lane / (BK / 8);
    const int row = min(m0 + rl, mlim - 1);   // rows past the segment: any valid row
    const int chunk = (lane % (BK / 8)) ^ kc_swz<BK>(rl);
    uint32_t o;
    if constexpr (KIND == KIND_FWD1 || KIND == KIND_DGRAD2) o = (uint32_t)(a.s2f[row] / k) * H;
    else if constexpr (KIND == KIND_FWD2) o = (uint32_t)row * I;
    else o = (uint32_t)row * 2 * I;
    return (o + chunk * 8) * 2;
  };
  auto b_kc_off = [&](int ci) __attribute__((always_inline)) -> uint32_t {
    const int nl = (512 / BK) * ci + lane / (BK / 8);
    const int chunk = (lane % (BK / 8)) ^ kc_swz<BK>(nl);
    uint32_t o;
    if constexpr (KIND == KIND_FWD1) {
      const int c = min(n0 + (nl & (BN / 2 - 1)), I - 1);
      o = (uint32_t)((nl < BN / 2) ? c : I + c) * H;
    } else {
      o = (uint32_t)min(n0 + nl, H - 1) * I;
    }
    return (o + chunk * 8) * 2;
  };
  uint32_t oa[DA], ob[DB];   // KC: byte offset of row + logical chunk; KO: byte offset of the columns
  int ka[K_::a_ko ? DA : 1], kb[K_::b_ko ? DB : 1];   // KO: k-row of the chunk inside the tile
#pragma unroll
  for (int i = 0; i < DA; ++i) {
    const int ci = i * NW + w_uni;
    if constexpr (!K_::a_ko) {
      oa[i] = a_kc_off(ci);
    } else {
      const int p = 1024 * ci + 16 * lane;
      const int kk = p / (BM * 2), byte = p % (BM * 2);
      const int col = ((((byte >> 5) ^ ko_f<BM>(kk))) << 4) + ((byte >> 4) & 1) * 8;
      ka[i] = kk;
      oa[i] = min(m0 + col, mlim - 8) * 2;
    }
  }
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int ci = i * NW + w_uni;
    if constexpr (!K_::b_ko) {
      ob[i] = b_kc_off(ci);
    } else {
      const int p = 1024 * ci + 16 * lane;
      const int kk = p / (BN * 2), byte = p % (BN * 2);
      const int col = ((((byte >> 5) ^ ko_f<BN>(kk))) << 4) + ((byte >> 4) & 1) * 8;
      kb[i] = kk;
      ob[i] = min(n0 + col, nlim - 8) * 2;
    }
  }

  // token offsets of gathered rows [klo + base, klo + base + TOKTAB)
  auto fill_tok = [&](int base) {
    for (int j = tid; j < TOKTAB; j += NTHR) {
      const int r = min(klo + base + j, khi - 1);
      s_tok[j] = (uint32_t)(a.s2f[r] / k) * H;
    }
  };

  const uint32_t lds0 = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)smem;
  // DMA instruction q (< DA + DB) of K tile kt into stage st (tiles past the
  // end read zeros): q < DA fills A-tile block q * NW + w, the rest B-tile blocks
  auto src_off = [&](int kt, int q) __attribute__((always_inline)) -> uint32_t {
    const bool live = kt < nk;
    if (q < DA) {
      const int i = q;
      if constexpr (!K_::a_ko) {
        return live ? oa[i] + (uint32_t)kt * (BK * 2) : OOB;
      } else {
        const int rr = kt * BK + ka[i];
        if constexpr (KIND == KIND_WGRAD2) {   // dY rows of the gathered tokens
          const uint32_t t = s_tok[rr & (TOKTAB - 1)];
          return (klo + rr < khi) ? t * 2 + oa[i] : OOB;
        } else {                               // dG13 rows
          return (klo + rr < khi) ? (uint32_t)(klo + rr) * (2 * I * 2) + oa[i] : OOB;
        }
      }
    } else {
      const int i = q - DA;
      if constexpr (!K_::b_ko) {
        return live ? ob[i] + (uint32_t)kt * (BK * 2) : OOB;
      } else if constexpr (K_::ragged_rows) {  // weights, dense K rows
        return live ? (uint32_t)(kt * BK + kb[i]) * (KIND == KIND_DGRAD2 ? I * 2 : H * 2) + ob[i] : OOB;
      } else {
        const int rr = kt * BK + kb[i];
        if constexpr (KIND == KIND_WGRAD2) {   // Ag rows
          return (klo + rr < khi) ? (uint32_t)(klo + rr) * (I * 2) + ob[i] : OOB;
        } else {                               // x rows of the gathered tokens
          const uint32_t t = s_tok[rr & (TOKTAB - 1)];
          return (klo + rr < khi) ? t * 2 + ob[i] : OOB;
        }
      }
    }
  };
  // byte offset in a stage of the 1 KiB block that instruction q of this wave fills
  auto blk_off = [&](int q) __attribute__((always_inline)) -> uint32_t {
    return q < DA ? (uint32_t)((q * NW + w_uni) * 1024) : (uint32_t)(BM * BK * 2 + ((q - DA) * NW + w_uni) * 1024);
  };
  // DMA instruction q (< DA + DB) of K tile kt into stage st (tiles past the
  // end read zeros)
  auto issue_one = [&](int kt, int st, int q) __attribute__((always_inline)) {
    const uint32_t sbase = lds0 + (uint32_t)(st * STAGE * 2);
    dma16(q < DA ? ra_src : rb_src, src_off(kt, q), __builtin_amdgcn_readfirstlane(sbase + blk_off(q)));
  };
  auto issue_tile = [&](int kt, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < DA + DB; ++q) issue_one(kt, st, q);
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

  // All MFMA operands of one K tile are read into registers first, so the
  // tile's LDS stage can be refilled while the MFMAs run.
  typedef bf16x8_t AFrag[BK / 32][FM];
  typedef bf16x8_t BFrag[BK / 32][FN];
  auto load_frags = [&](int st, AFrag& af, BFrag& bfr) __attribute__((always_inline)) {
    const bf16_t* As = smem + st * STAGE;
    const bf16_t* Bs = As + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (K_::a_ko) af[ks][i] = frag_ko<BM>(As, wm * WM + 16 * i, ks, lane);
        else af[ks][i] = frag_kc<BK>(As, wm * WM + 16 * i, ks, lane);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (K_::b_ko) bfr[ks][j] = frag_ko<BN>(Bs, brow(j), ks, lane);
        else bfr[ks][j] = frag_kc<BK>(Bs, brow(j), ks, lane);
      }
    }
  };
  // The MFMAs of one tile with the DMA of tile kt into stage st spread
  // between them (one DMA instruction every NM / ND MFMAs), so that the
  // address queue drains while the matrix cores work.
  auto mfmas_dma = [&](const AFrag& af, const BFrag& bfr, int kt, int st) __attribute__((always_inline)) {
    constexpr int NM = (BK / 32) * FM * FN, ND = DA + DB;
    constexpr int SP = NM / ND > 0 ? NM / ND : 1;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int idx = (ks * FM + i) * FN + j;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[ks][j], af[ks][i], acc[i][j], 0, 0, 0);
          if (idx % SP == SP - 1 && idx / SP < ND) {
            issue_one(kt, st, idx / SP);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
    for (int q = NM / SP; q < ND; ++q) issue_one(kt, st, q);   // when there are more DMAs than MFMAs
  };
  // the token table of the gathered rows moves on when tile kl starts a new chunk
  auto refill_tok = [&](int kl) __attribute__((always_inline)) {
    if constexpr (gathered_k) {
      if ((kl * BK) % TOKTAB == 0 && kl < nk) {
        fill_tok(kl * BK);
        __syncthreads();
      }
    }
  };

  // ---------------- main loop ----------------
  if constexpr (gathered_k) {
    if (nk > 0) { fill_tok(0); __syncthreads(); }
  }
  // A wave whose rows all lie past the expert's end (the ragged last tile)
  // computes nothing it would store: it keeps its share of the DMA and the
  // barriers and skips its fragment reads and MFMAs.
  const bool idle = K_::ragged_rows && __builtin_amdgcn_readfirstlane((int)(m0 + wm * WM >= mlim)) != 0;
  if constexpr (C::PIPE == 2) {
    // Ping-pong between the two wave rows, P (row 0) and Q (row 1); each SIMD
    // holds one wave of each.  Block barriers split the loop into phases: P
    // reads its fragments of K tile t in phase 2t and multiplies them in
    // phase 2t+1, Q reads them in phase 2t+1 and multiplies them in phase
    // 2t+2, so that in every phase one wave of a SIMD feeds the matrix core
    // while the other waits on the LDS.  Each group loads the half of the A
    // tile that only it reads, during its MFMAs; Q also loads the B tile,
    // ahead of its A half, since P reads it one phase earlier.  A stage is
    // free once Q has read it (phase 2t+1), so tile t+2 lands in the stage of
    // tile t: P's half from phase 2t+1, Q's part from phase 2t+2.
    static_assert(C::WGM == 2 && S == 2 && !K_::a_ko && K_::ragged_rows,
                  "ping-pong main loop: row kinds with a K-contiguous A, two wave rows, two stages");
    constexpr int NG = NW / 2;                          // waves per group
    constexpr int PA = (BM / 2) * BK * 2 / 1024 / NG;   // DMAs per wave and tile: its group's half of A
    constexpr int PB = BN * BK * 2 / 1024 / NG;         // DMAs per Q wave and tile: the B tile
    static_assert(PA * NG * 1024 == (BM / 2) * BK * 2 && PB * NG * 1024 == BN * BK * 2, "1 KiB DMA blocks");
    const bool gq = w_uni / C::WGN == 1;                // wave row 1 (uniform: from the read-first-lane wave index)
    const int wg = w_uni % NG;
    const int a_blk0 = (gq ? PA * NG : 0) + wg;         // first A-tile block of this wave
    uint32_t pa[PA], pb[PB];
    int pkb[K_::b_ko ? PB : 1];   // KO B: k-row of the block inside the tile
#pragma unroll
    for (int i = 0; i < PA; ++i) pa[i] = a_kc_off(a_blk0 + i * NG);
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int ci = i * NG + wg;
      if constexpr (!K_::b_ko) {
        pb[i] = b_kc_off(ci);
      } else {   // as the KO B offsets above
        const int p = 1024 * ci + 16 * lane;
        const int kk = p / (BN * 2), byte = p % (BN * 2);
        const int col = ((((byte >> 5) ^ ko_f<BN>(kk))) << 4) + ((byte >> 4) & 1) * 8;
        pkb[i] = kk;
        pb[i] = min(n0 + col, nlim - 8) * 2;
      }
    }
    auto dma_a = [&](int kt, int st, int i) __attribute__((always_inline)) {
      dma16(ra_src, kt < nk ? pa[i] + (uint32_t)kt * (BK * 2) : OOB,
            __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(st * STAGE * 2 + (a_blk0 + i * NG) * 1024)));
    };
    auto dma_b = [&](int kt, int st, int i) __attribute__((always_inline)) {
      uint32_t off;
      if constexpr (!K_::b_ko) off = pb[i] + (uint32_t)kt * (BK * 2);
      else off = (uint32_t)(kt * BK + pkb[i]) * (KIND == KIND_DGRAD2 ? I * 2 : H * 2) + pb[i];
      dma16(rb_src, kt < nk ? off : OOB,
            __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(st * STAGE * 2 + BM * BK * 2 + (i * NG + wg) * 1024)));
    };
    // Q's DMAs of a tile: the B tile first, then its A half
    auto dma_q = [&](int kt, int st, int q) __attribute__((always_inline)) {
      if (q < PB) dma_b(kt, st, q);
      else dma_a(kt, st, q - PB);
    };
    // a whole K tile's MFMAs with ND DMAs spread between them
    auto mfmas_spread = [&](const AFrag& af, const BFrag& bfr, auto nd, auto&& issue) __attribute__((always_inline)) {
      constexpr int NM = (BK / 32) * FM * FN, ND = decltype(nd)::value;
      constexpr int SP = NM / ND > 0 ? NM / ND : 1;
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int idx = (ks * FM + i) * FN + j;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[ks][j], af[ks][i], acc[i][j], 0, 0, 0);
            if (idx % SP == SP - 1 && idx / SP < ND) {
              issue(idx / SP);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
      for (int q = NM / SP; q < ND; ++q) issue(q);
    };
    auto phase_end = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // Both groups run "read tile t, barrier, multiply tile t, barrier" loops
    // with the same barrier count; Q's loop starts one phase later and P
    // passes one barrier more at the end.  One loop per group and per idle
    // state, so that no branch splits the MFMA stream.
    auto pp_loop = [&](auto q_c, auto idle_c) __attribute__((always_inline)) {
      constexpr bool GQ = decltype(q_c)::value, IDLE = decltype(idle_c)::value;
      constexpr int ND = GQ ? PB + PA : PA;   // DMAs per tile of this wave
      auto dma_tile = [&](int kt, int st, int q) __attribute__((always_inline)) {
        if constexpr (GQ) dma_q(kt, st, q);
        else dma_a(kt, st, q);
      };
      AFrag af;
      BFrag bfr;
#pragma unroll
      for (int q = 0; q < ND; ++q) dma_tile(0, 0, q);
#pragma unroll
      for (int q = 0; q < ND; ++q) dma_tile(1, 1, q);
      if constexpr (GQ) {
        vm_wait<2 * PA + PB>();   // the B tile of tile 0, before P reads it (phase 0)
        phase_end();
        vm_wait<PB + PA>();       // its A half of tile 0, before it reads it (phase 1)
      } else {
        vm_wait<PA>();            // its A half of tile 0
      }
      phase_end();
      for (int t = 0; t < nk; ++t) {
        const int st = t & 1;
        // read tile t (P: phase 2t, Q: phase 2t+1)
        if constexpr (!IDLE) {
          load_frags(st, af, bfr);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if constexpr (GQ) vm_wait<PA>();   // the B tile of tile t + 1, before P reads it
        phase_end();
        // multiply tile t; tile t + 2 into stage st (P: its A half in phase
        // 2t+1; Q: the B tile and its A half in phase 2t+2)
        if constexpr (!IDLE) {
          mfmas_spread(af, bfr, std::integral_constant<int, ND>{},
                       [&](int q) __attribute__((always_inline)) { dma_tile(t + 2, st, q); });
        } else {
#pragma unroll
          for (int q = 0; q < ND; ++q) dma_tile(t + 2, st, q);
        }
        vm_wait<GQ ? PB + PA : PA>();   // its A half of tile t + 1
        phase_end();
      }
      if constexpr (!GQ) phase_end();   // Q's last multiply
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (gq) {
      if (idle) pp_loop(T_{}, T_{});
      else pp_loop(T_{}, F_{});
    } else {
      if (idle) pp_loop(F_{}, T_{});
      else pp_loop(F_{}, F_{});
    }
  } else if constexpr (C::PIPE == 1) {
    // Software pipeline over 32-wide K steps: the fragments of the next step
    // are read from LDS while the MFMAs of the current one run.  One barrier
    // per K tile, before its last step: it publishes tile kt + 1 (every
    // wave's DMA of it has landed) and frees the stage of tile kt (every
    // wave has read its fragments), which then receives tile kt + S while the
    // last step's MFMAs run; the first step of tile kt + 1 is read meanwhile.
    constexpr int KS = BK / 32, ND = DA + DB;
    typedef bf16x8_t AStep[FM];
    typedef bf16x8_t BStep[FN];
    auto read_step = [&](int st, int ks, AStep& a_, BStep& b_) __attribute__((always_inline)) {
      const bf16_t* As = smem + st * STAGE;
      const bf16_t* Bs = As + BM * BK;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (K_::a_ko) a_[i] = frag_ko<BM>(As, wm * WM + 16 * i, ks, lane);
        else a_[i] = frag_kc<BK>(As, wm * WM + 16 * i, ks, lane);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (K_::b_ko) b_[j] = frag_ko<BN>(Bs, brow(j), ks, lane);
        else b_[j] = frag_kc<BK>(Bs, brow(j), ks, lane);
      }
      __builtin_amdgcn_sched_barrier(0);   // the reads go out before the MFMAs they overlap
    };
    auto mfma_step = [&](const AStep& a_, const BStep& b_) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b_[j], a_[i], acc[i][j], 0, 0, 0);
    };
    // the last step's MFMAs with the DMA of tile kt into stage st spread between them
    auto mfma_step_dma = [&](const AStep& a_, const BStep& b_, int kt, int st) __attribute__((always_inline)) {
      constexpr int NM = FM * FN;
      constexpr int SP = NM / ND > 0 ? NM / ND : 1;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int idx = i * FN + j;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b_[j], a_[i], acc[i][j], 0, 0, 0);
          if (idx % SP == SP - 1 && idx / SP < ND) {
            issue_one(kt, st, idx / SP);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
      for (int q = NM / SP; q < ND; ++q) issue_one(kt, st, q);
    };
    // lgkmcnt(0) as a builtin (vmcnt and expcnt fields at their maxima), so
    // that the compiler knows every LDS read has completed
    auto lds_wait_all = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0xC07F); };

#pragma unroll
    for (int st = 0; st < S; ++st) issue_tile(st, st);
    vm_wait<(S - 1) * ND>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int st_c = 0;
    // the barrier of tile kt: this wave's reads of the tile are complete and
    // its DMA of tile kt + 1 has landed, then the block synchronises
    auto publish = [&](int kt) __attribute__((always_inline)) {
      lds_wait_all();
      vm_wait<(S - 2) * ND>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      refill_tok(kt + S);
    };
    if (idle) {   // the same barriers and DMA, no reads or MFMAs
      for (int kt = 0; kt < nk; ++kt) {
        publish(kt);
        issue_tile(kt + S, st_c);
        st_c = (st_c + 1 == S) ? 0 : st_c + 1;
      }
    } else if constexpr (KS == 2) {
      AStep a0, a1;
      BStep b0, b1;
      read_step(0, 0, a0, b0);
      for (int kt = 0; kt < nk; ++kt) {
        const int st_n = (st_c + 1 == S) ? 0 : st_c + 1;
        read_step(st_c, 1, a1, b1);         // step 1 of this tile
        mfma_step(a0, b0);                  // step 0
        publish(kt);
        read_step(st_n, 0, a0, b0);         // step 0 of the next tile
        mfma_step_dma(a1, b1, kt + S, st_c);   // step 1, refilling this tile's stage
        st_c = st_n;
      }
    } else {
      AStep a0, a1;
      BStep b0, b1;
      read_step(0, 0, a0, b0);
      for (int kt = 0; kt < nk; kt += 2) {
        const int s1 = (st_c + 1 == S) ? 0 : st_c + 1;
        publish(kt);
        read_step(s1, 0, a1, b1);
        mfma_step_dma(a0, b0, kt + S, st_c);
        st_c = s1;
        if (kt + 1 < nk) {
          const int s2 = (st_c + 1 == S) ? 0 : st_c + 1;
          publish(kt + 1);
          read_step(s2, 0, a0, b0);
          mfma_step_dma(a1, b1, kt + 1 + S, st_c);
          st_c = s2;
        }
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < S; ++st) issue_tile(st, st);
    // S tiles in flight.  Iteration kt: wait for this wave's DMA of tile kt; a
    // barrier publishes it; every wave reads its operands into registers; a
    // second barrier frees the stage, which receives tile kt + S while the
    // MFMAs run from registers.
    AFrag af;
    BFrag bfr;
    int st_c = 0;
    if (idle) {
      for (int kt = 0; kt < nk; ++kt) {
        vm_wait<(S - 1) * (DA + DB)>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_tile(kt + S, st_c);
        st_c = (st_c + 1 == S) ? 0 : st_c + 1;
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) {
        vm_wait<(S - 1) * (DA + DB)>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        load_frags(st_c, af, bfr);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        refill_tok(kt + S);
        mfmas_dma(af, bfr, kt + S, st_c);
        st_c = (st_c + 1 == S) ? 0 : st_c + 1;
      }
    }
  }
  vm_wait<0>();      // no DMA may land while the epilogue reuses LDS
  __syncthreads();

  gg::gemm_epilogue<KIND, C>(a, acc, smem, tid, lane, wm, wn, e, m0, mlim, n0, nlim, wout, wacc);
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

// Tile shapes (BM x BN, waves WGM x WGN, waves per SIMD, LDS stages, K tile,
// tile-group divisor, main loop).  Forward: 256 x 256 tiles with a 64-wide K
// tile (128-byte rows per DMA lane group, one 8-wave block per CU): fewer
// operand bytes per flop and full cache lines outweigh the longer ragged tail
// (measured 8 % faster for both forward GEMMs); tile groups of 8 blocks, a
// quarter of an XCD's resident blocks (about 2 % faster than 32); the
// ping-pong loop (GEMM W13 6 % faster at the 30B shape, 11 % at the 235B
// shape, GEMM W2 1 % and 5 %).  The dgrad kinds measured faster with
// 128 x 256, K tile 32, two 4-wave blocks per CU, and whole-XCD tile groups.
#ifndef MOE_CFG_ROW_FWD
#define MOE_CFG_ROW_FWD 256, 256, 2, 4, 2, 2, 64, 4, 2
#endif
#ifndef MOE_CFG_ROW
#define MOE_CFG_ROW 128, 256, 2, 2, 2, 2, 32
#endif
// dgrad kinds when both of their K dimensions (H for W2, 2I for W13) reach
// MOE_DGRAD_LONG_K: 256 x 256 tiles with the ping-pong loop, whose fixed
// start and end phases then weigh less (Qwen3-235B-A22B shape: dgrad W13
// 3.26 -> 2.96 ms, dgrad W2 1.92 -> 1.79 ms; at the 30B shape, K = 2048 and
// 1536, the same tiles were 0-5 % slower than two 128 x 256 blocks per CU)
#ifndef MOE_CFG_ROW_LONG
#define MOE_CFG_ROW_LONG 256, 256, 2, 4, 2, 2, 64, 4, 2
#endif
#ifndef MOE_DGRAD_LONG_K
#define MOE_DGRAD_LONG_K 3072
#endif
// Weight gradients: two 4-wave blocks per CU (57 KB of LDS each), so that
// one block's fp32 output stores overlap the other's main loop.  wgrad of W2
// (M = H, N = I): 128 x 256, wgrad of W13 (M = 2I, N = H): 256 x 128; against
// one 8-wave 256 x 256 block per CU, 1-2 % and 3 % faster with the even
// routing, 4 % and 7 % with the skewed one.
#ifndef MOE_CFG_WGRAD
#define MOE_CFG_WGRAD 128, 256, 2, 2, 2, 2, 32
#endif
#ifndef MOE_CFG_WGRAD1
#define MOE_CFG_WGRAD1 256, 128, 2, 2, 2, 2, 32
#endif
using CfgRowF = TileCfg<MOE_CFG_ROW_FWD>;
using CfgRow = TileCfg<MOE_CFG_ROW>;
using CfgRowL = TileCfg<MOE_CFG_ROW_LONG>;
static_assert(CfgRowL::BN == CfgRow::BN, "one gate-gradient partial per 256-column tile of the dgrad of W2");
using CfgW = TileCfg<MOE_CFG_WGRAD>;
using CfgW1 = TileCfg<MOE_CFG_WGRAD1>;

template <int KIND, class C>
hipError_t launch_kind(const LayerArgs& a, hipStream_t s) {
  int n_tiles, tiles;
  if constexpr (Kind<KIND>::ragged_rows) {
    const int ncols = (KIND == KIND_FWD1) ? a.I : (KIND == KIND_FWD2 || KIND == KIND_DGRAD1) ? a.H : a.I;
    const int bn = (KIND == KIND_FWD1) ? C::BN / 2 : C::BN;
    n_tiles = (ncols + bn - 1) / bn;
    tiles = n_tiles * max_row_tiles(a.M, a.E, C::BM);
  } else {
    const int mdim = (KIND == KIND_WGRAD2) ? a.H : 2 * a.I;
    const int ndim = (KIND == KIND_WGRAD2) ? a.I : a.H;
    n_tiles = (ndim + C::BN - 1) / C::BN;
    tiles = a.E * n_tiles * ((mdim + C::BM - 1) / C::BM);
  }
  const int nvb = Kind<KIND>::ragged_rows ? (tiles + NXCD - 1) / NXCD * NXCD
                                          : wgrad_grid(wgrad_max_chunks(a.M, a.E), tiles / a.E);
  const int grid = C::PERSIST ? min(nvb, resident_blocks(C::WPE * 4 / C::NW)) : nvb;
  return launch_kernel((gemm_bf16_kernel<KIND, C>), dim3(grid), dim3(C::NTHR), 0, s, a, n_tiles, tiles, nvb);
}

}  // namespace

int bf16_fwd_row_tile_m() { return CfgRowF::BM; }
bool bf16_dgrad_long(int H, int I) { return H >= MOE_DGRAD_LONG_K && 2 * I >= MOE_DGRAD_LONG_K; }
int bf16_row_tile_m(int H, int I) { return bf16_dgrad_long(H, I) ? CfgRowL::BM : CfgRow::BM; }
int bf16_dgrad2_tile_n() { return CfgRow::BN; }

hipError_t launch_gemm_bf16(GemmKind kind, const LayerArgs& a, hipStream_t s) {
  const bool long_k = bf16_dgrad_long(a.H, a.I);
  switch (kind) {
    case KIND_FWD1: return launch_kind<KIND_FWD1, CfgRowF>(a, s);
    case KIND_FWD2: return launch_kind<KIND_FWD2, CfgRowF>(a, s);
    case KIND_DGRAD2: return long_k ? launch_kind<KIND_DGRAD2, CfgRowL>(a, s) : launch_kind<KIND_DGRAD2, CfgRow>(a, s);
    case KIND_DGRAD1: return long_k ? launch_kind<KIND_DGRAD1, CfgRowL>(a, s) : launch_kind<KIND_DGRAD1, CfgRow>(a, s);
    case KIND_WGRAD2: return launch_kind<KIND_WGRAD2, CfgW>(a, s);
    case KIND_WGRAD1: return launch_kind<KIND_WGRAD1, CfgW1>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
