// FP8 (E4M3) grouped expert GEMMs on gfx950.
//
// GEMMs in FP8 with fine-grained scaling: activations carry one fp32 scale per
// 1x128 tile (per token, 128 channels), weights one per 128x128 block, and
// partial products are promoted to fp32 at every 128-wide slice of the
// contraction (mhpq.cn "DeepSeek-V3 高效训练关键技术全景解析" §4.1; gkm0120.cn
// DeepSeek-V3 notes, Q8). Here one LDS stage holds exactly one 128-wide slice,
// so two chained v_mfma_scale_f32_32x32x64_f8f6f4 (unit hardware scales, k 0-63
// then 64-127) yield the slice's exact-product partial sum for a 32x32
// sub-tile; the fp32 scale product s_a(row) * s_b(block) is applied on the
// VALU as it is accumulated. The 32x32x64 operand pattern (32 rows x two
// 32-byte k groups per wave) reads LDS without bank conflicts; the 16x16x128
// one (16 rows x four k groups) is two-way conflicted under any chunk swizzle.
//
// The gate/up GEMM covers 128 intermediate columns per tile, i.e. exactly one
// 1x128 quantization tile of H: its epilogue computes silu(gate) * up, the
// row max-abs across the tile's waves, and writes E4M3 codes plus the fp32
// scale that the down GEMM consumes.
#pragma clang fp contract(off)

#include "device_common.h"
#include "internal.h"
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
  // loads per thread and k block: A and B tiles, one row scale, two block scales
  static constexpr int NL = A_LOADS + B_LOADS + 3;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "waves cover whole 32x32 products");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must cover the load passes");
  static_assert(BM <= NT, "one thread per row loads the activation scales");
  static_assert(NST >= 3 && NL * (NST - 2) <= 63, "ring depth within the vmcnt range");
};

using T8Gate = Tile8<128, 256, 64, 64>;        // 8 waves, H tile 128 x 128, 144 KB ring
using T8Down = Tile8<128, 256, 64, 64>;        // 8 waves, 144 KB ring
using T8GateDec = Tile8<32, 256, 32, 64, 4, true>;   // 4 waves, 144 KB ring
using T8DownDec = Tile8<32, 128, 32, 64, 6, true>;   // 2 waves, 120 KB ring

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
// wave's own slot of lds_sb. Every wave issues the same number of loads per
// k block, so one vmcnt bound holds for all of them.
template <class C>
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
  dma4(op.rsa, op.sa_off + kb4, __builtin_amdgcn_readfirstlane(sa0 + (st * C::NT + wave * 64) * 4));
  const uint32_t sb_base =
      __builtin_amdgcn_readfirstlane(sb0 + ((st * C::NWAVES + wave) * 2) * 4);
  if (lane == 0) {
    dma4(op.rsb, op.sb_lo + kb4, sb_base);
    dma4(op.rsb, op.sb_hi + kb4, sb_base + 4);
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
template <class C, bool SWIGLU, class Mid>
__device__ __forceinline__ void stage8_mma(const uint8_t* lds, const float* lds_sa,
                                           const float* lds_sb, int st, int wave, int wm, int wn,
                                           int lane, f32x16_t (&acc)[C::MI][C::NJ], Mid&& mid) {
  const uint8_t* As = lds + st * C::STAGE;
  const uint8_t* Bs = As + C::BM * BK8;
  const float s_lo = lds_sb[(st * C::NWAVES + wave) * 2];
  const float s_hi = SWIGLU ? lds_sb[(st * C::NWAVES + wave) * 2 + 1] : s_lo;
  const int rl = lane & 31;
  const int ch = 2 * (lane >> 5);  // first chunk of the lane's 32-byte k group
  float sl[C::MI], sh[C::MI];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    const float sa = lds_sa[st * C::NT + wm * C::WM + mi * 32 + rl];
    sl[mi] = sa * s_lo;
    sh[mi] = sa * s_hi;
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
    const float s = (!SWIGLU || pn < C::NJ / 2) ? sl[pm] : sh[pm];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[pm][pn][r] = __builtin_fmaf(p[u & 1][r], s, acc[pm][pn][r]);
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
    p[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[nj][0], af[mi & 1][0], zero, 0,
                                                               0, 0, 127, 0, 127);
    p[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[nj][1], af[mi & 1][1],
                                                               p[t & 1], 0, 0, 0, 127, 0, 127);
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
template <class C, bool SWIGLU, class NextOps, class NkOf, class Epilogue>
__device__ __forceinline__ void gemm8_stream(uint8_t* lds, float* lds_sa, float* lds_sb, int first,
                                             int nb, int total, NextOps&& next_ops, NkOf&& nk_of,
                                             Epilogue&& epilogue) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  constexpr int NST = C::NST;
  constexpr int INFLIGHT = C::NL * (NST - 2);
  const uint32_t lds0 = lds_addr(lds), sa0 = lds_addr(lds_sa), sb0 = lds_addr(lds_sb);

  // issue side
  StreamOps8<C> op;
  int ti = first, ki = 0, index = 0;
  bool more = true;
  next_ops(ti, index, op);
  auto issue = [&](int st) {
    stage8_issue<C>(lds0, sa0, sb0, st, wave, lane, op, ki);
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
  auto mid = [&]() {
    vm_wait<INFLIGHT>();
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
      issue(st_issue);  // into the stage read in the previous k block
      advance();
      stage8_mma<C, SWIGLU>(lds, lds_sa, lds_sb, st, wave, wm, wn, lane, acc, mid);
      st = st == NST - 1 ? 0 : st + 1;
      st_issue = st_issue == NST - 1 ? 0 : st_issue + 1;
    }
    epilogue(tc, acc);
  }
  // the reloads past the last block land before the workgroup ends
  vm_wait<0>();
}

// H (E4M3 + 1x128 scales) = quant(silu(A W1^T) * (A W3^T)); tile = 128 H
// columns. Routed rows of A are gathered through perm: the token indices of a
// tile's rows come into an LDS slot by the same asynchronous loads as the
// operands, one tile ahead, so that the tile loop issues no compiler-visible
// global loads.
template <class C>
__global__ __launch_bounds__(C::NT, 2) void ffn1_fp8_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_sa[C::NST * C::NT];
  __shared__ __attribute__((aligned(16))) float lds_sb[C::NST * C::NWAVES * 2];
  __shared__ float red[C::WAVES_N][C::BM];
  __shared__ GroupTables gt;
  constexpr int PS = C::BM > 64 ? C::BM : 64;  // one dma4 per 64 rows
  __shared__ __attribute__((aligned(16))) int pslot[2][PS];
  constexpr int HALF = C::BN / 2;  // 128 H columns
  static_assert(HALF == 128, "one 1x128 quantization tile of H per tile");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles1, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const int dkb = a.d / 128;
  const int hkb = a.ldh / 128;
  const float* XS = a.perm ? a.x_scale : a.xperm_scale;
  const i32x4_t rxs = rsrc4(a.x, static_cast<uint32_t>(a.T) * static_cast<uint32_t>(a.d));
  const i32x4_t rx =
      a.perm ? rxs : rsrc4(a.xperm, static_cast<uint32_t>(a.TK) * static_cast<uint32_t>(a.d));
  // activation scales: gathered rows (or x_perm rows) and the shared rows
  const i32x4_t rsxp =
      rsrc4(XS, static_cast<uint32_t>(a.perm ? a.T : a.TK) * static_cast<uint32_t>(dkb) * 4u);
  const i32x4_t rsx =
      rsrc4(a.x_scale, static_cast<uint32_t>(a.T) * static_cast<uint32_t>(dkb) * 4u);
  const i32x4_t rperm = rsrc4(a.perm, static_cast<uint32_t>(a.TK) * 4u);
  const int nk = a.d / BK8;
  uint8_t* H = static_cast<uint8_t*>(a.H);

  // token indices of a routed tile's rows into slot s (rows past the group
  // are masked where they are used)
  auto fetch_perm = [&](int tile, int s) {
    if (!a.perm || wave * 64 >= C::BM) return;
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    if (c.shared) return;
    const int j = wave * 64 + lane;
    const uint32_t off =
        j < C::BM ? static_cast<uint32_t>(c.rbase + c.m * C::BM + j) * 4u : kInvalidRow;
    dma4(rperm, off, __builtin_amdgcn_readfirstlane(lds_addr(&pslot[s][wave * 64])));
  };
  fetch_perm(first, 0);
  if (first + nb < total) fetch_perm(first + nb, 1);
  vm_wait<0>();
  lds_barrier();

  auto next_ops = [&](int tile, int index, StreamOps8<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int* slot = pslot[index & 1];
    if (index > 0) {
      // slot index & 1 was filled while tile index - 1 was issued, nk blocks
      // ago: landed once NST - 2 further blocks of loads were issued after it
      if (nk < C::NST - 1) {
        vm_wait<0>();
        lds_barrier();
      }
      if (tile + nb < total) fetch_perm(tile + nb, (index + 1) & 1);
    }
    const int Ig = c.shared ? a.Is : a.I;
    // source row (token) of tile row r, or -1
    auto src_row = [&](int r) -> int {
      const int gr = c.m * C::BM + r;
      if (gr >= c.rows) return -1;
      if (c.shared) return gr;
      if (a.perm) {
        const int tok = slot[r];
        return (tok >= 0 && tok < a.T) ? tok : -1;
      }
      return c.rbase + gr;
    };
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int row = src_row(r0 + p * C::RPP);
      op.ao[p] = row >= 0 ? static_cast<uint32_t>(row) * static_cast<uint32_t>(a.d) : kInvalidRow;
    }
    op.sa_off = kInvalidRow;
    if (tid < C::BM) {
      const int row = src_row(tid);
      if (row >= 0) op.sa_off = static_cast<uint32_t>(row * dkb) * 4u;
    }
    op.ra = c.shared ? rxs : rx;
    op.rsa = c.shared ? rsx : rsxp;
    const uint8_t* W = c.shared ? static_cast<const uint8_t*>(a.ws13)
                                : static_cast<const uint8_t*>(a.w13) +
                                      static_cast<int64_t>(c.g) * 2 * a.I * a.d;
    const float* WS = c.shared ? a.ws13_scale
                               : a.w13_scale + static_cast<int64_t>(c.g) * (2 * a.I / 128) * dkb;
    op.rb = rsrc4(W, static_cast<uint32_t>(2 * Ig) * a.d);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      const bool up = lr >= HALF;
      const int col = c.n * HALF + (up ? lr - HALF : lr);
      op.bo[p] = static_cast<uint32_t>(up ? Ig + col : col) * static_cast<uint32_t>(a.d);
    }
    op.rsb = rsrc4(WS, static_cast<uint32_t>(2 * Ig / 128) * static_cast<uint32_t>(dkb) * 4u);
    op.sb_lo = static_cast<uint32_t>(c.n * dkb) * 4u;
    op.sb_hi = static_cast<uint32_t>((Ig / 128 + c.n) * dkb) * 4u;
    swizzle_rows8<C>(op.ao);
    swizzle_rows8<C>(op.bo);
    op.nk = nk;
  };
  auto nk_of = [&](int) { return nk; };
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    // SwiGLU, then the row max-abs over the 128 columns: lane l holds 16 of
    // the 32 columns of row l % 32 in each product, lane l ^ 32 the other 16,
    // and the tile's WAVES_N waves the rest of the row
    constexpr int NJH = C::NJ / 2;
    float h[C::MI][NJH][16];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      float m = 0.0f;
#pragma unroll
      for (int nj = 0; nj < NJH; ++nj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          h[mi][nj][r] = silu_f32(acc[mi][nj][r]) * acc[mi][nj + NJH][r];
          m = fmaxf(m, fabsf(h[mi][nj][r]));
        }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (lane < 32) red[wn][wm * C::WM + mi * 32 + lane] = m;
    }
    lds_barrier();
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    const int rows_left = c.rows - c.m * C::BM;
    // E4M3 codes leave straight from registers, four columns per 4-byte store
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int lr = wm * C::WM + mi * 32 + (lane & 31);
      float amax = red[0][lr];
#pragma unroll
      for (int w = 1; w < C::WAVES_N; ++w) amax = fmaxf(amax, red[w][lr]);
      if (lr >= rows_left) continue;
      const float inv = amax == 0.0f ? 0.0f : 448.0f / amax;
      uint8_t* hp = H + (hrow0 + lr) * a.ldh + c.n * HALF + wn * (C::WN / 2) + 4 * (lane >> 5);
#pragma unroll
      for (int nj = 0; nj < NJH; ++nj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float* v = &h[mi][nj][4 * g];
          *reinterpret_cast<uint32_t*>(hp + nj * 32 + 8 * g) =
              amax == 0.0f ? 0u : e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        }
      if (wn == 0 && lane < 32)
        a.H_scale[(hrow0 + lr) * hkb + c.n] = amax == 0.0f ? 1.0f : amax / 448.0f;
    }
    // red[] is rewritten by the next tile's epilogue only after at least one
    // more k block, whose barrier orders these reads first
  };
  gemm8_stream<C, true>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of, epilogue);
}

// y = dequant(H) dequant(W2)^T per group, bf16 out, stored from registers.
template <class C>
__global__ __launch_bounds__(C::NT, 2) void ffn2_fp8_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_sa[C::NST * C::NT];
  __shared__ __attribute__((aligned(16))) float lds_sb[C::NST * C::NWAVES * 2];
  __shared__ GroupTables gt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles2, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const int hkb = a.ldh / 128;
  const int64_t hrows = a.TK + (a.Is > 0 ? a.T : 0);
  const i32x4_t rh = rsrc4(a.H, static_cast<uint32_t>(hrows) * static_cast<uint32_t>(a.ldh));
  const i32x4_t rsh =
      rsrc4(a.H_scale, static_cast<uint32_t>(hrows) * static_cast<uint32_t>(hkb) * 4u);
  // the shared group's tiles are the last ones
  const int shared_first = a.E > 0 ? gt.gnext[a.E - 1] : 0;
  // weight block scales of a wave's WN output columns (inside one 128-row
  // block of W2)
  static_assert(128 % C::WN == 0, "a wave's columns lie in one scale block");

  auto next_ops = [&](int tile, int, StreamOps8<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    const int rows_left = c.rows - c.m * C::BM;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left
                     ? static_cast<uint32_t>(hrow0 + lr) * static_cast<uint32_t>(a.ldh)
                     : kInvalidRow;
    }
    op.sa_off = (tid < C::BM && tid < rows_left) ? static_cast<uint32_t>((hrow0 + tid) * hkb) * 4u
                                                 : kInvalidRow;
    op.ra = rh;
    op.rsa = rsh;
    const uint8_t* W = c.shared ? static_cast<const uint8_t*>(a.ws2)
                                : static_cast<const uint8_t*>(a.w2) +
                                      static_cast<int64_t>(c.g) * a.d * a.I;
    const int ikb = Ig / 128;
    const float* WS = c.shared ? a.ws2_scale
                               : a.w2_scale + static_cast<int64_t>(c.g) * (a.d / 128) * (a.I / 128);
    op.rb = rsrc4(W, static_cast<uint32_t>(a.d) * static_cast<uint32_t>(Ig));
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = c.n * C::BN + r0 + p * C::RPP;
      op.bo[p] = row < a.d ? static_cast<uint32_t>(row) * static_cast<uint32_t>(Ig) : kInvalidRow;
    }
    op.rsb = rsrc4(WS, static_cast<uint32_t>(a.d / 128) * static_cast<uint32_t>(ikb) * 4u);
    op.sb_lo = op.sb_hi =
        static_cast<uint32_t>(((c.n * C::BN + wn * C::WN) / 128) * ikb) * 4u;
    swizzle_rows8<C>(op.ao);
    swizzle_rows8<C>(op.bo);
    op.nk = Ig / BK8;
  };
  auto nk_of = [&](int tile) { return (tile >= shared_first ? a.Is : a.I) / BK8; };
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int rows_left = c.rows - c.m * C::BM;
    uint16_t* out = c.shared ? static_cast<uint16_t*>(a.yshared) +
                                   static_cast<int64_t>(c.m) * C::BM * a.d
                             : static_cast<uint16_t*>(a.yperm) +
                                   (static_cast<int64_t>(c.rbase) + c.m * C::BM) * a.d;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int row = wm * C::WM + mi * 32 + (lane & 31);
      if (row >= rows_left) continue;
      uint16_t* yp = out + static_cast<int64_t>(row) * a.d;
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = c.n * C::BN + wn * C::WN + nj * 32 + 8 * g + 4 * (lane >> 5);
          if (col >= a.d) continue;
          const f32x16_t& v = acc[mi][nj];
          *reinterpret_cast<uint2*>(yp + col) = make_uint2(pack_bf16x2(v[4 * g], v[4 * g + 1]),
                                                           pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
        }
    }
  };
  gemm8_stream<C, false>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of, epilogue);
}

template <class K>
int occupancy8(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

template <class C1, class C2>
hipError_t launch_fp8_pair(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  static int occ1 = 0, occ2 = 0;
  if (!occ1) occ1 = occupancy8(ffn1_fp8_kernel<C1>, C1::NT);
  if (!occ2) occ2 = occupancy8(ffn2_fp8_kernel<C2>, C2::NT);
  const int cus = device_cu_count();
  const int g1 = ((cus * occ1 + 7) / 8) * 8;
  const int g2 = ((cus * occ2 + 7) / 8) * 8;
  hipLaunchKernelGGL(ffn1_fp8_kernel<C1>, dim3(g1), dim3(C1::NT), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(ffn2_fp8_kernel<C2>, dim3(g2), dim3(C2::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

GemmTiling choose_tiling_fp8(double rows_per_expert) {
  GemmTiling t{};
  if (rows_per_expert < 48.0) {
    t.bm1 = T8GateDec::BM; t.bnh1 = T8GateDec::BN / 2;
    t.bm2 = T8DownDec::BM; t.bn2 = T8DownDec::BN; t.variant = 1;
  } else {
    t.bm1 = T8Gate::BM; t.bnh1 = T8Gate::BN / 2;
    t.bm2 = T8Down::BM; t.bn2 = T8Down::BN; t.variant = 0;
  }
  return t;
}

hipError_t launch_ffn_fp8(const FfnArgs& a, const GemmTiling& t, hipStream_t s, hipEvent_t mid) {
  if (t.variant == 1) return launch_fp8_pair<T8GateDec, T8DownDec>(a, s, mid);
  return launch_fp8_pair<T8Gate, T8Down>(a, s, mid);
}

}  // namespace dsmoe
