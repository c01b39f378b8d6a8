// FP8 k-stream core shared by the grouped FP8 GEMMs of the layer (forward
// gate/up and down projections, the backward's input- and weight-gradient
// products): tile shapes, the swizzled LDS layout, LDS-DMA issue of code
// tiles and scales, the per-128-k-block MFMA step with its fp32 scale fold,
// and the persistent one-k-stream-per-workgroup loop. Everything here is in an
// anonymous namespace, so each translation unit gets its own copy.
//
// Scaling (mhpq.cn "DeepSeek-V3 高效训练关键技术全景解析" §4.1; gkm0120.cn
// DeepSeek-V3 notes, Q8): one fp32 scale per 128-wide slice of the
// contraction on each side, so one LDS stage holds exactly one slice and two
// chained v_mfma_scale_f32_32x32x64_f8f6f4 (unit hardware scales, k 0-63 then
// 64-127) give the slice's exact-product partial sum, which the VALU scales
// and adds in fp32.
#pragma once

#include "device_common.h"
#include "tile_schedule.h"

namespace dsmoe {
namespace {

constexpr int BK8 = 128;  // E4M3 elements (bytes) per row per stage = one scale block

// BM x BN tile in waves of WM x WN; NST LDS stages in the load ring (loads run
// NST - 1 k blocks ahead). B_NT: weight tiles are loaded with the
// non-temporal policy (decode, where each weight slab is read by one tile;
// where several m-tiles of an expert share a slab through L2 it costs 30%).
template <int BM_, int BN_, int WM_, int WN_, int NST_ = 3, bool B_NT_ = false>
struct Tile8 {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NST = NST_;
  static constexpr bool B_NT = B_NT_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int RPP = NT / 8;
  static constexpr int A_LOADS = BM / RPP;
  static constexpr int B_LOADS = BN / RPP;
  static constexpr int STAGE = (BM + BN) * BK8;  // bytes
  static constexpr int LDS_BYTES = NST * STAGE;
  // vector-memory instructions per wave and k block: A and B tiles, one row
  // scale, and two block scales (lane 0) or, with row scales for B too, one
  // more per-thread row scale
  template <bool SBROW>
  static constexpr int NL = A_LOADS + B_LOADS + (SBROW ? 2 : 3);
  static_assert(WM % 32 == 0 && WN % 32 == 0, "waves cover whole 32x32 products");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must cover the load passes");
  static_assert(BM <= NT && BN <= NT, "one thread per row loads the row scales");
  static_assert(NST >= 3 && (A_LOADS + B_LOADS + 3) * (NST - 2) <= 63,
                "ring depth within the vmcnt range");
};


// Byte offset of 16-byte chunk `ch` of row `r`, swizzled with (r >> 1) & 7 so
// that the 32 rows x 2 chunks one 128-bit fragment read serves spread over all
// 64 banks.
__device__ __forceinline__ int lds_off8(int r, int ch) {
  return r * BK8 + ((ch ^ ((r >> 1) & 7)) << 4);
}

template <class C, bool SWIGLU>
__device__ __forceinline__ int b_row8(int wn, int nj) {
  if constexpr (SWIGLU) {
    constexpr int half = C::BN / 2, hw = C::WN / 2, njh = C::NJ / 2;
    return nj < njh ? wn * hw + nj * 32 : half + wn * hw + (nj - njh) * 32;
  } else {
    return wn * C::WN + nj * 32;
  }
}

// 32 bytes of row r: chunks ch and ch + 1
__device__ __forceinline__ i32x8_t frag8(const uint8_t* tile, int r, int ch) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + lds_off8(r, ch));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + lds_off8(r, ch + 1));
  i32x8_t v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// Operands of one tile's k-stream: buffer resources, per-thread row byte
// offsets (swizzle folded in), this thread's activation-scale row offset, the
// weight block-scale offsets of the wave's gate (lo) and up (hi) columns, and
// the number of 128-wide k blocks.
template <class C>
struct StreamOps8 {
  i32x4_t ra, rsa, rb, rsb;
  uint32_t ao[C::A_LOADS], bo[C::B_LOADS];
  uint32_t sa_off, sb_lo, sb_hi;
  uint32_t sb_off;  // row scales for B (SBROW): this thread's B row
  // bytes between the A row scales of consecutive k blocks: 4 for scales
  // stored row-major, the row count for k-block-major scales (a tile's row
  // scales of one k block are then contiguous)
  uint32_t sa_step = 4;
  uint32_t sb_step = 4;  // the same for the B row scales (SBROW)
  int nk;
};

// Folds the chunk swizzle into the row offsets: lane (row r, 16-byte position
// ch) fetches logical chunk ch ^ swizzle(r), giving the layout lds_off8 reads.
template <class C, int N>
__device__ __forceinline__ void swizzle_rows8(uint32_t (&o)[N]) {
  const int ch = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
  for (int p = 0; p < N; ++p)
    o[p] += static_cast<uint32_t>((ch ^ (((r0 + p * C::RPP) >> 1) & 7)) * 16);
}

// Issues k block kb of a tile into ring stage st. All loads go from global
// memory straight into LDS: the code tiles with 16-byte loads, the row scales
// with one 4-byte load per lane into lds_sa[stage][thread] (zeros past the
// tile's rows), the two block scales with lane-0-only 4-byte loads into the
// wave's own slot of lds_sb, or, with SBROW (B has one scale per row and k
// block), one 4-byte load per lane into lds_sb[stage][thread]. Every wave
// issues the same number of loads per k block, so one vmcnt bound holds for
// all of them.
template <class C, bool SBROW = false>
__device__ __forceinline__ void stage8_issue(uint32_t lds0, uint32_t sa0, uint32_t sb0, int st,
                                             int wave, int lane, const StreamOps8<C>& op,
                                             int kb) {
  const uint32_t off = static_cast<uint32_t>(kb) * BK8;
  const uint32_t a_base = __builtin_amdgcn_readfirstlane(lds0 + st * C::STAGE + wave * 8 * BK8);
  const uint32_t b_base = a_base + C::BM * BK8;
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) dma16(op.ra, op.ao[p] + off, a_base + p * C::RPP * BK8);
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) {
    if constexpr (C::B_NT)
      dma16_nt(op.rb, op.bo[p] + off, b_base + p * C::RPP * BK8);
    else
      dma16(op.rb, op.bo[p] + off, b_base + p * C::RPP * BK8);
  }
  const uint32_t kb4 = static_cast<uint32_t>(kb) * 4u;
  dma4(op.rsa, op.sa_off + static_cast<uint32_t>(kb) * op.sa_step,
       __builtin_amdgcn_readfirstlane(sa0 + (st * C::NT + wave * 64) * 4));
  if constexpr (SBROW) {
    dma4(op.rsb, op.sb_off + static_cast<uint32_t>(kb) * op.sb_step,
         __builtin_amdgcn_readfirstlane(sb0 + (st * C::NT + wave * 64) * 4));
  } else {
    const uint32_t sb_base =
        __builtin_amdgcn_readfirstlane(sb0 + ((st * C::NWAVES + wave) * 2) * 4);
    if (lane == 0) {
      dma4(op.rsb, op.sb_lo + kb4, sb_base);
      dma4(op.rsb, op.sb_hi + kb4, sb_base + 4);
    }
  }
}

// acc[mi][nj] += (A_kb B_kb^T) * s_a[row][kb] * s_b[kb] for the k block in
// ring stage st (s_b: the gate block for the first half of the wave's column
// sub-tiles, the up block for the second; one block without SWIGLU). The
// weight fragment goes first: lane l then owns token row l % 32 of each
// 32-row group and 16 columns of each 32x32 product (columns 8g + 4(l / 32)
// + q, g and q below 4), so one row-scale x block-scale product serves all 16
// values of a product. A product is two MFMAs (k 0-63, then 64-127 onto the
// first's result, in the matrix core). Products are pipelined one deep:
// product t's MFMAs run while the VALU folds product t-1 into its
// accumulator. mid() runs once every LDS read of the stage has been issued,
// before the last row group's MFMAs, whose operands are then in registers.
// FW / FA: formats of the B (weight-side, first MFMA operand) and A codes,
// 0 = E4M3, 1 = E5M2. SBROW: B carries one scale per row and k block instead
// of a block scale, so each of a lane's 16 values gets its own scale product.
// SWAP = false (SBROW only) puts the A fragment first instead: lane l then
// owns B row (output column) l % 32 and the 16 A rows 8 g + 4 (l / 32) + q of
// each 32-row group, so that one accumulator register across the wave is two
// 128-byte output row pieces (full cache lines for fp32 outputs).
template <class C, bool SWIGLU, int FW, int FA, bool SBROW, bool SWAP, class Mid>
__device__ __forceinline__ void stage8_mma(const uint8_t* lds, const float* lds_sa,
                                           const float* lds_sb, int st, int sbw, int wm, int wn,
                                           int lane, f32x16_t (&acc)[C::MI][C::NJ], Mid&& mid) {
  static_assert(SWAP || SBROW, "the A-first order is built for row scales on both sides");
  const uint8_t* As = lds + st * C::STAGE;
  const uint8_t* Bs = As + C::BM * BK8;
  const float s_lo = SBROW ? 1.0f : lds_sb[(st * C::NWAVES + sbw) * 2];
  const float s_hi = SBROW ? 1.0f : SWIGLU ? lds_sb[(st * C::NWAVES + sbw) * 2 + 1] : s_lo;
  const int rl = lane & 31;
  const int ch = 2 * (lane >> 5);  // first chunk of the lane's 32-byte k group
  float sl[C::MI], sh[C::MI];
  if constexpr (SWAP) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const float sa = lds_sa[st * C::NT + wm * C::WM + mi * 32 + rl];
      sl[mi] = sa * s_lo;
      sh[mi] = sa * s_hi;
    }
  }
  // SBROW: the scales of the lane's 16 rows on the register side (B rows
  // with SWAP, A rows without) and of its one row on the lane side, read
  // now: after mid()'s barrier the stage's scale slots may already be
  // refilled for a later k block
  constexpr int NR = SWAP ? C::NJ : C::MI;
  float sbv[SBROW ? NR : 1][16];
  float slane[SWAP ? 1 : C::NJ];
  if constexpr (SBROW) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float* sr = SWAP ? lds_sb + st * C::NT + b_row8<C, SWIGLU>(wn, i) + 4 * (lane >> 5)
                             : lds_sa + st * C::NT + wm * C::WM + i * 32 + 4 * (lane >> 5);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 s4 = *reinterpret_cast<const float4*>(sr + 8 * g);
        sbv[i][4 * g] = s4.x;
        sbv[i][4 * g + 1] = s4.y;
        sbv[i][4 * g + 2] = s4.z;
        sbv[i][4 * g + 3] = s4.w;
      }
    }
    if constexpr (!SWAP) {
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
        slane[nj] = lds_sb[st * C::NT + b_row8<C, SWIGLU>(wn, nj) + rl];
    }
  }
  i32x8_t bfr[C::NJ][2];
#pragma unroll
  for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      bfr[nj][h] = frag8(Bs, b_row8<C, SWIGLU>(wn, nj) + rl, 4 * h + ch);
  auto a_frag = [&](int m, int h) { return frag8(As, wm * C::WM + m * 32 + rl, 4 * h + ch); };
  constexpr int NP = C::MI * C::NJ;
  constexpr int TMID = (C::MI - 1) * C::NJ;  // first product of the last row group
  f32x16_t p[2];
  i32x8_t af[2][2];
  af[0][0] = a_frag(0, 0);
  af[0][1] = a_frag(0, 1);
  auto fold = [&](int u) {
    const int pm = u / C::NJ, pn = u % C::NJ;
    if constexpr (SBROW && SWAP) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[pm][pn][r] = __builtin_fmaf(p[u & 1][r], sl[pm] * sbv[pn][r], acc[pm][pn][r]);
    } else if constexpr (SBROW) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[pm][pn][r] = __builtin_fmaf(p[u & 1][r], sbv[pm][r] * slane[pn], acc[pm][pn][r]);
    } else {
      const float s = (!SWIGLU || pn < C::NJ / 2) ? sl[pm] : sh[pm];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[pm][pn][r] = __builtin_fmaf(p[u & 1][r], s, acc[pm][pn][r]);
    }
  };
#pragma unroll
  for (int t = 0; t < NP; ++t) {
    const int mi = t / C::NJ, nj = t % C::NJ;
    if (t == TMID) {
      __builtin_amdgcn_sched_barrier(0);
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
    const f32x16_t zero = {};
    if constexpr (SWAP) {
      p[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[nj][0], af[mi & 1][0], zero,
                                                                 FW, FA, 0, 127, 0, 127);
      p[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[nj][1], af[mi & 1][1],
                                                                 p[t & 1], FW, FA, 0, 127, 0, 127);
    } else {
      p[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi & 1][0], bfr[nj][0], zero,
                                                                 FA, FW, 0, 127, 0, 127);
      p[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi & 1][1], bfr[nj][1],
                                                                 p[t & 1], FA, FW, 0, 127, 0, 127);
    }
    if (nj == 0 && mi + 1 < C::MI) {
      af[(mi + 1) & 1][0] = a_frag(mi + 1, 0);
      af[(mi + 1) & 1][1] = a_frag(mi + 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t > 0) fold(t - 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  fold(NP - 1);
}

// The persistent FP8 GEMMs run every tile of a workgroup (tiles first,
// first + nb, ... below total) as one k-stream through the NST-stage ring:
// the first k blocks of a tile are loaded during the previous tile's last
// ones, so the ring never drains at a tile boundary.
//   next_ops(tile, index, ops): operands of the index-th tile of the issue
//     side (called once per tile, in order, after the previous tile's last
//     k block was issued);
//   nk_of(tile): k blocks of a tile;
//   epilogue(tile, acc): stores a finished tile.
// Vector-memory waits count only this stream's loads: every k block issues
// the same loads (once the tiles run out, the last block is loaded again into
// stages nobody reads), so with loads NST - 1 blocks ahead at most the newest
// NL * (NST - 2) may be in flight when a stage is read; extra loads or stores
// in between only make such a wait stronger.
// POST >= 0 lets the epilogue's stores drain during the next tile's first
// two k blocks: the next tile's first loads are issued before the epilogue
// (into the stage the last block has just freed), so the stages both of
// those blocks wait for were loaded before the stores, and their waits
// allow POST operations in flight instead. With NST = 3, one k block's loads
// and the epilogue's stores follow each of those stages, so that is exact
// only if every epilogue call issues at least POST - NL vector-memory
// instructions. SWAP: operand order of the MFMAs (stage8_mma).
template <class C, bool SWIGLU, class NextOps, class NkOf, class Epilogue, int FW = 0, int FA = 0,
          bool SBROW = false, bool SWAP = true, int POST = -1>
__device__ __forceinline__ void gemm8_stream(uint8_t* lds, float* lds_sa, float* lds_sb, int first,
                                             int nb, int total, NextOps&& next_ops, NkOf&& nk_of,
                                             Epilogue&& epilogue, int sb_wave = -1) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // block scales (no SBROW): the wave whose slot holds this wave's two
  // scales (waves with the same scales let one of them load them; the
  // others' scale loads read out of range and fetch nothing)
  const int sbw = sb_wave < 0 ? wave : sb_wave;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  constexpr int NST = C::NST;
  constexpr int INFLIGHT = C::template NL<SBROW> * (NST - 2);
  const uint32_t lds0 = lds_addr(lds), sa0 = lds_addr(lds_sa), sb0 = lds_addr(lds_sb);
  static_assert(POST < 0 || NST == 3, "the early issue before an epilogue assumes three stages");

  // issue side
  StreamOps8<C> op;
  int ti = first, ki = 0, index = 0;
  bool more = true;
  next_ops(ti, index, op);
  auto issue = [&](int st) {
    stage8_issue<C, SBROW>(lds0, sa0, sb0, st, wave, lane, op, ki);
    if (more) ++ki;
  };
  auto advance = [&]() {
    if (!more || ki < op.nk) return;
    ki = 0;
    ti += nb;
    if (ti < total) {
      next_ops(ti, ++index, op);
    } else {
      more = false;
      ki = op.nk - 1;
    }
  };
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) {
    issue(j);
    advance();
  }
  vm_wait<INFLIGHT>();  // stage 0 has landed
  lds_barrier();

  // compute side
  int st = 0, st_issue = NST - 1;
  // this wave's part of the next stage has landed; the barrier makes every
  // wave's part visible and frees the stage being read
  bool after_epilogue = false;
  auto mid = [&]() {
    if constexpr (POST >= 0) {
      static_assert(POST >= INFLIGHT && POST <= 63, "vmcnt range");
      if (after_epilogue)
        vm_wait<POST>();
      else
        vm_wait<INFLIGHT>();
    } else {
      vm_wait<INFLIGHT>();
    }
    lds_barrier();
  };
  for (int tc = first; tc < total; tc += nb) {
    f32x16_t acc[C::MI][C::NJ];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) acc[mi][nj] = f32x16_t{};
    const int nkc = nk_of(tc);
    for (int kc = 0; kc < nkc; ++kc) {
      // into the stage read in the previous k block (with POST, the first
      // block's loads went out before the previous tile's epilogue)
      if (POST < 0 || kc > 0 || tc == first) {
        issue(st_issue);
        advance();
      }
      after_epilogue = POST >= 0 && kc < 2 && tc != first;
      stage8_mma<C, SWIGLU, FW, FA, SBROW, SWAP>(lds, lds_sa, lds_sb, st, sbw, wm, wn, lane, acc,
                                                 mid);
      st = st == NST - 1 ? 0 : st + 1;
      st_issue = st_issue == NST - 1 ? 0 : st_issue + 1;
    }
    if constexpr (POST >= 0) {
      if (tc + nb < total) {
        issue(st_issue);
        advance();
      }
    }
    epilogue(tc, acc);
  }
  // the reloads past the last block land before the workgroup ends
  vm_wait<0>();
}

}  // namespace
}  // namespace dsmoe
