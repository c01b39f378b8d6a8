// bf16 k-stream core shared by the grouped GEMMs of the layer: tile shapes,
// the swizzled LDS layout, LDS-DMA stage issue and the persistent
// one-k-stream-per-workgroup loop (see gemm_stream). Included by the
// translation units of the forward and backward GEMMs; everything here is in
// an anonymous namespace, so each gets its own copy.
#pragma once

#include "device_common.h"
#include "tile_schedule.h"

namespace dsmoe {
namespace {

constexpr int BK = 64;  // k elements per stage: 128 bytes per row

// BM x BN output tile in waves of WM x WN; NST LDS stages in the load ring
// (loads run NST - 1 k-steps ahead). B_NT: B tiles are loaded with the
// non-temporal policy: decode streams each weight slab through one tile, and
// there it reads 13-18% faster; where several m-tiles of an expert share a
// slab through L2 (prefill, the backward) it costs 30%.
template <int BM_, int BN_, int WM_, int WN_, int NST_ = 3, bool B_NT_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NST = NST_;
  static constexpr bool B_NT = B_NT_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int RPP = NT / 8;  // rows covered by one pass of 16-byte loads
  static constexpr int A_LOADS = BM / RPP;
  static constexpr int B_LOADS = BN / RPP;
  static constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per stage
  // waves per SIMD the register budget is sized for
  static constexpr int MINW = (WM * WN >= 64 * 128) ? 1 : 2;
  static constexpr int LDS_ELEMS = NST * STAGE;
  static_assert(NST >= 2, "loads run at least one step ahead");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must cover the load passes");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA sub-tiles");
};

using TilePrefill = Tile<128, 256, 64, 64>;  // 8 waves, 144 KB LDS
// decode streams weights: one 2-wave workgroup per CU with a 7-stage ring
// keeps six steps (120 KB) of loads in flight per CU
using TileDecode = Tile<32, 128, 32, 64, 7, true>;

// LDS element offset of 16-byte chunk `ch` (0..7) of row `r`. The chunk is
// XOR-swizzled with (r >> 1) & 7: the 16 lanes that one 128-bit LDS access
// serves together read 16 consecutive rows at one logical chunk, and with two
// 128-byte rows per 64-bank line this spreads them over all 64 banks.
__device__ __forceinline__ int lds_off(int r, int ch) {
  return r * BK + ((ch ^ ((r >> 1) & 7)) << 3);
}

template <class C, bool SWIGLU>
__device__ __forceinline__ int b_local_row(int wn, int nj) {
  if constexpr (SWIGLU) {
    constexpr int half = C::BN / 2, hw = C::WN / 2, njh = C::NJ / 2;
    return nj < njh ? wn * hw + nj * 32 : half + wn * hw + (nj - njh) * 32;
  } else {
    return wn * C::WN + nj * 32;
  }
}

// Global byte offsets of one thread's rows with the chunk swizzle folded in:
// lane (row r, 16-byte position ch) fetches logical chunk ch ^ swizzle(r), so
// the LDS image of a stage is the swizzled layout lds_off describes.
template <class C, int N>
__device__ __forceinline__ void swizzle_rows(uint32_t (&o)[N]) {
  const int ch = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
  for (int p = 0; p < N; ++p)
    o[p] += static_cast<uint32_t>((ch ^ (((r0 + p * C::RPP) >> 1) & 7)) * 16);
}

// Issues one k-step of A and B rows (byte offsets ao, bo plus ka, kb) from
// global memory straight into ring stage st: no registers hold tiles in flight
// and no LDS store instructions are issued. This wave's 8 rows of each load
// pass start at row 8 * wave.
template <class C>
__device__ __forceinline__ void stage_issue(uint32_t lds0, int st, int wave, i32x4_t ra,
                                            const uint32_t (&ao)[C::A_LOADS], uint32_t ka,
                                            i32x4_t rb, const uint32_t (&bo)[C::B_LOADS],
                                            uint32_t kb) {
  const uint32_t a_base =
      __builtin_amdgcn_readfirstlane(lds0 + (st * C::STAGE + wave * 8 * BK) * 2);
  const uint32_t b_base = a_base + C::BM * BK * 2;
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) dma16(ra, ao[p] + ka, a_base + p * C::RPP * BK * 2);
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) {
    if constexpr (C::B_NT)
      dma16_nt(rb, bo[p] + kb, b_base + p * C::RPP * BK * 2);
    else
      dma16(rb, bo[p] + kb, b_base + p * C::RPP * BK * 2);
  }
}


template <class C>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[C::MI][C::NJ]) {
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;
}

// loads of the NST - 2 newest steps that may stay in flight at a wait
template <class C>
constexpr int kInflight = (C::A_LOADS + C::B_LOADS) * (C::NST - 2);


// Operands of one tile's k-stream: buffer resources, per-thread row byte
// offsets (swizzle folded in) and the number of 64-wide k-steps.
template <class C>
struct StreamOps {
  i32x4_t ra, rb;
  uint32_t ao[C::A_LOADS], bo[C::B_LOADS];
  int nk;
  uint32_t kstep_a, kstep_b;  // k-major operands only: bytes between k-steps
};

// ---- k-major operands ([K, N] row-major: the k-step is BK consecutive rows)
//
// Stage image of a k-major operand of width W (BN for B, BM for A): BK rows
// (k) of W elements; 16-byte chunk c of row k sits at position c ^ (4 (k & 3)).
// Every load pass keeps the LDS placement of the row-major stage (one
// 16-byte chunk per thread, threads in order), so only the thread ->
// (k, chunk) assignment differs: thread t of pass p loads row
// p * (NT * 8 / W) + t / (W / 8), logical chunk (t % (W / 8)) ^ (4 (row & 3)).
//
// Fragments come from ds_read_b64_tr_b16: in each 16-lane group, lane i
// receives element i % 4 of the 8-byte pieces that lanes 4j + i / 4
// (j = 0..3) address. With lane 4j + q of the group pointing at row k + j,
// columns n + 4q .. n + 4q + 3, lane i gets column n + i at rows k .. k + 3;
// two reads give the 8 consecutive k of a 32x32x16 MFMA operand. The
// swizzle puts the four rows of one read on distinct banks.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Global byte offsets of thread t's chunks of a k-major operand of width W
// for k-step 0 (row r of the step at r * ld_bytes; `col0` is the tile's
// first column); LOADS passes of NT threads.
template <int W, int LOADS, int NT>
__device__ __forceinline__ void kmajor_offsets(uint32_t (&o)[LOADS], int col0, uint32_t ld_bytes) {
  constexpr int CPR = W / 8, RPASS = NT / CPR;
  static_assert(NT % CPR == 0 && LOADS * RPASS == BK, "passes cover the k-step");
  const int t = threadIdx.x;
  const int row = t / CPR;
  const uint32_t chunk = static_cast<uint32_t>((t % CPR) ^ (4 * (row & 3)));
#pragma unroll
  for (int p = 0; p < LOADS; ++p)
    o[p] = static_cast<uint32_t>(p * RPASS + row) * ld_bytes +
           static_cast<uint32_t>(col0 + chunk * 8) * 2u;
}

// The MFMA operand of columns [n0, n0 + 32) and k [k0, k0 + 16) (lane l:
// column n0 + l % 32, k0 + 8 (l / 32) .. + 7) from a k-major stage of width
// W at LDS byte address base.
template <int W>
__device__ __forceinline__ bf16x8_t frag_kmajor(uint32_t base, int n0, int k0, int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  const int n = n0 + 16 * (g & 1) + 4 * q;
  const int k = k0 + 8 * (g >> 1) + j;
  const int chunk = (n >> 3) ^ (4 * j);  // k & 3 == j
  const uint32_t a0 = base + static_cast<uint32_t>(k * W + chunk * 8 + (n & 4)) * 2u;
  const uint32_t a1 = a0 + 4u * W * 2u;  // rows k + 4: same swizzle
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a0);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a1);
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// The persistent grouped GEMMs run every tile of a workgroup (tiles first,
// first + nb, ... below total) as one k-stream through the NST-stage ring:
// the first steps of a tile are loaded during the previous tile's last
// steps, so the ring never drains at a tile boundary, and a tile's epilogue
// (stores straight from registers, no LDS) runs while the next tile's first
// stages land.
//   next_ops(tile, index, ops): operands of the index-th tile of the issue
//     side (called once per tile, in order, after the previous tile's last
//     step was issued);
//   nk_of(tile): k-steps of a tile;
//   epilogue(tile, acc): stores a finished tile. With SWAP (the default) the
//     weight fragment goes first and acc holds the transposed tile: lane l
//     owns output row l % 32 and, per group of four registers, four adjacent
//     columns; without it lane l owns output column l % 32 and rows
//     acc_row(l, r), so that one register across the wave is two 128-byte
//     row pieces (full cache lines for fp32 outputs).
// BKM / AKM: B / A is k-major (offsets from kmajor_offsets, advanced by
// ops.kstep_b / ops.kstep_a per k-step, fragments by transpose reads).
// POST >= 0 lets the epilogue's stores drain during the next tile's first
// step: that step's wait allows POST operations in flight instead of
// kInflight<C>, which is exact only if every epilogue call issues at least
// POST - kInflight<C> vector-memory instructions (the stage that step needs
// was loaded before them).
// Vector-memory waits count only this stream's loads: every step issues the
// same loads (once the tiles run out, the last step is loaded again into
// stages nobody reads), so with loads NST - 1 steps ahead at most the newest
// kInflight<C> may be in flight when a stage is read; extra loads or stores
// issued in between only make such a wait stronger.
// Within a step, the fragments of sub-step kk + 1 are read while sub-step kk
// multiplies; the step's barrier sits before its last sub-step, whose
// fragments are already in registers, so that the next stage's first
// fragments are read while those MFMAs run.
// rows_of(tile) (optional): rows of the tile that hold data (the rest are
// padding past a group's last row). A wave whose 64-row band holds fewer
// rows skips the MFMAs of its 32-row sub-tiles that lie wholly past them:
// the count is fixed per tile, so each count runs its own copy of the k-loop
// and no branch splits a step (the fragment reads stay as they are, so the
// registers that carry the next tile's first sub-step are always filled).
struct AllRows {
  __device__ int operator()(int) const { return 1 << 30; }
};
template <int N>
struct IntC {
  static constexpr int value = N;
};

template <class C, bool SWIGLU, class NextOps, class NkOf, class Epilogue, bool SWAP = true,
          int POST = -1, bool BKM = false, bool AKM = false, class RowsOf = AllRows>
__device__ __forceinline__ void gemm_stream(uint16_t* lds, int first, int nb, int total,
                                            NextOps&& next_ops, NkOf&& nk_of,
                                            Epilogue&& epilogue, RowsOf rows_of = RowsOf{}) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  constexpr int NST = C::NST;
  constexpr int INFLIGHT = kInflight<C>;
  static_assert(INFLIGHT <= 63, "vmcnt range");
  static_assert(BK / 16 == 4, "four MFMA sub-steps per k-step");
  // with two stages the next tile's first waited stage is loaded after the
  // epilogue's stores, so they cannot drain past that wait
  static_assert(POST < 0 || NST >= 3, "POST needs loads two steps ahead");
  const uint32_t lds0 = lds_addr(lds);

  // issue side
  StreamOps<C> op;
  int ti = first, ki = 0, index = 0;
  bool more = true;
  next_ops(ti, index, op);
  auto issue = [&](int st) {
    const uint32_t kn = static_cast<uint32_t>(ki) * (BK * 2);
    const uint32_t ka = AKM ? static_cast<uint32_t>(ki) * op.kstep_a : kn;
    const uint32_t kb = BKM ? static_cast<uint32_t>(ki) * op.kstep_b : kn;
    stage_issue<C>(lds0, st, wave, op.ra, op.ao, ka, op.rb, op.bo, kb);
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

  // fragments of sub-step kk of stage st
  bf16x8_t af[2][C::MI], bfr[2][C::NJ];
  auto fetch = [&](int st, int kk, int buf) {
    const uint16_t* As = lds + st * C::STAGE;
    const uint16_t* Bs = As + C::BM * BK;
    const int chk = kk * 2 + (lane >> 5);
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) {
      if constexpr (BKM)
        bfr[buf][nj] =
            frag_kmajor<C::BN>(lds_addr(Bs), b_local_row<C, SWIGLU>(wn, nj), kk * 16, lane);
      else
        bfr[buf][nj] = *reinterpret_cast<const bf16x8_t*>(
            Bs + lds_off(b_local_row<C, SWIGLU>(wn, nj) + (lane & 31), chk));
    }
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      if constexpr (AKM)
        af[buf][mi] = frag_kmajor<C::BM>(lds_addr(As), wm * C::WM + mi * 32, kk * 16, lane);
      else
        af[buf][mi] = *reinterpret_cast<const bf16x8_t*>(
            As + lds_off(wm * C::WM + mi * 32 + (lane & 31), chk));
    }
  };
  f32x16_t acc[C::MI][C::NJ];
  auto mma = [&](int buf, auto nmi) {
#pragma unroll
    for (int mi = 0; mi < decltype(nmi)::value; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) {
        if constexpr (SWAP)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][nj], af[buf][mi],
                                                                acc[mi][nj], 0, 0, 0);
        else
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][mi], bfr[buf][nj],
                                                                acc[mi][nj], 0, 0, 0);
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
  fetch(st, 0, 0);
  for (int tc = first; tc < total; tc += nb) {
    zero_acc<C>(acc);
    const int nkc = nk_of(tc);
    auto kloop = [&](auto nmi) {
    for (int kc = 0; kc < nkc; ++kc) {
      issue(st_issue);  // into the stage read in the previous step
      fetch(st, 1, 1);
      // fragment reads go out before the MFMAs that do not need them (the
      // scheduler would otherwise reuse their registers and serialize)
      __builtin_amdgcn_sched_barrier(0);
      mma(0, nmi);
      advance();
      fetch(st, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      mma(1, nmi);
      fetch(st, 3, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(0, nmi);
      // this wave's part of the next stage has landed; the barrier makes
      // every wave's part visible and frees the stage whose last fragments
      // are now in registers
      if constexpr (POST >= 0) {
        static_assert(POST >= INFLIGHT && POST <= 63, "vmcnt range");
        if (kc == 0 && tc != first)
          vm_wait<POST>();
        else
          vm_wait<INFLIGHT>();
      } else {
        vm_wait<INFLIGHT>();
      }
      lds_barrier();
      st = st == NST - 1 ? 0 : st + 1;
      st_issue = st_issue == NST - 1 ? 0 : st_issue + 1;
      fetch(st, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mma(1, nmi);
    }
    };
    // 32-row sub-tiles of this wave's band that hold data
    const int band = rows_of(tc) - wm * C::WM;
    const int nmi = band <= 0 ? 0 : band >= C::WM ? C::MI : (band + 31) / 32;
    static_assert(C::MI <= 4, "row-skip counts 0..4");
    if (nmi >= C::MI) {
      kloop(IntC<C::MI>{});
    } else if constexpr (C::MI == 1) {
      kloop(IntC<0>{});
    } else {
      if constexpr (C::MI >= 4) {
        if (nmi == 3) { kloop(IntC<3 % C::MI>{}); epilogue(tc, acc); continue; }
      }
      if constexpr (C::MI >= 3) {
        if (nmi == 2) { kloop(IntC<2 % C::MI>{}); epilogue(tc, acc); continue; }
      }
      if (nmi == 1)
        kloop(IntC<1>{});
      else
        kloop(IntC<0>{});
    }
    epilogue(tc, acc);
  }
  // the reloads past the last step land before the workgroup ends
  vm_wait<0>();
}

// Row (within the tile) of accumulator element r of a 32x32 sub-tile, for
// this lane; the lane's column is lane % 32.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}


}  // namespace
}  // namespace dsmoe
