// bf16 MFMA GEMMs of the layer on gfx950:
//   - the grouped expert GEMMs: [gate; up] projection with the SwiGLU
//     epilogue, then the down projection, for every routed expert's segment
//     plus the shared expert, which applies to every token (mhpq.cn
//     "DeepSeek-V3 高效训练关键技术全景解析" §1.1);
//   - the router product in exact-input fp32: the fp32 router weights are
//     split into three bf16 terms hi + mid + lo that sum to them exactly, so
//     every bf16(x) * term product is exact and the sum is accumulated in fp32
//     (the gating module stays in high precision, same article §4.1).
//
// Tiles are staged through LDS with an XOR swizzle (conflict-free 16-byte
// fragment reads), double-buffered so one barrier per 64-wide k step suffices,
// and multiplied with v_mfma_f32_32x32x16_bf16. The grouped GEMMs run as
// persistent kernels over a device-built tile list, with workgroups remapped
// so that consecutive tiles (which share weight or activation panels) run on
// the same XCD and hit in its L2.
#include "device_common.h"
#include "internal.h"
#include "tile_schedule.h"

namespace dsmoe {

namespace {

constexpr int BK = 64;  // k elements per stage: 128 bytes per row

// BM x BN output tile in waves of WM x WN; NST LDS stages in the load ring
// (loads run NST - 1 k-steps ahead).
template <int BM_, int BN_, int WM_, int WN_, int NST_ = 3>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NST = NST_;
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
  static_assert(NST >= 3, "loads run at least two steps ahead");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must cover the load passes");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA sub-tiles");
};

using TilePrefill = Tile<128, 256, 64, 64>;  // 8 waves, 144 KB LDS
// decode streams weights: one 2-wave workgroup per CU with a 7-stage ring
// keeps six steps (120 KB) of loads in flight per CU
using TileDecode = Tile<32, 128, 32, 64, 7>;

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

// acc[mi][nj] += A * B^T over k in [k_begin, k_end) (multiples of 64).
// Operands come from buffers (ra, rb) through a 32-bit byte offset per thread
// and row (the k = 0 element of the row); offsets at or beyond the buffer
// size (kInvalidRow) read as zeros, so padding rows cost no branches. With
// a_kmod != 0 the A column is k mod a_kmod (router: the same activations meet
// the three weight terms). Padding rows are multiplied as zeros.
//
// Tiles go from global memory straight into a ring of NST LDS stages,
// NST - 1 k-steps ahead, with one barrier per step: no registers hold tiles in
// flight and no LDS store instructions are issued. Lane (row r, 16-byte
// position ch) fetches logical chunk ch ^ swizzle(r), so the LDS image is the
// swizzled layout lds_off describes. Within a step, the LDS fragments of the
// next 16-wide sub-step are read while the current one multiplies.
template <class C, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(uint16_t* lds, i32x4_t ra,
                                          const uint32_t (&aoff)[C::A_LOADS], i32x4_t rb,
                                          const uint32_t (&boff)[C::B_LOADS], int k_begin,
                                          int k_end, int a_kmod, f32x16_t (&acc)[C::MI][C::NJ]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int ch = tid & 7, r0 = tid >> 3;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;
  uint32_t ao[C::A_LOADS], bo[C::B_LOADS];
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p)
    ao[p] = aoff[p] + static_cast<uint32_t>((ch ^ (((r0 + p * C::RPP) >> 1) & 7)) * 16);
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p)
    bo[p] = boff[p] + static_cast<uint32_t>((ch ^ (((r0 + p * C::RPP) >> 1) & 7)) * 16);
  const uint32_t lds0 = lds_addr(lds);
  // this wave's 8 rows of each load pass start at row 8 * wave
  auto issue = [&](int st, int k0) {
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
    const uint32_t ka = a_kmod ? static_cast<uint32_t>(k0 % a_kmod) * 2u : kb;
    const uint32_t a_base =
        __builtin_amdgcn_readfirstlane(lds0 + (st * C::STAGE + wave * 8 * BK) * 2);
    const uint32_t b_base = a_base + C::BM * BK * 2;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) dma16(ra, ao[p] + ka, a_base + p * C::RPP * BK * 2);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) dma16(rb, bo[p] + kb, b_base + p * C::RPP * BK * 2);
  };
  auto compute = [&](int st) {
    const uint16_t* As = lds + st * C::STAGE;
    const uint16_t* Bs = As + C::BM * BK;
    bf16x8_t af[2][C::MI], bfr[2][C::NJ];
    auto fetch = [&](int kk, int buf) {
      const int chk = kk * 2 + (lane >> 5);
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
        bfr[buf][nj] = *reinterpret_cast<const bf16x8_t*>(
            Bs + lds_off(b_local_row<C, SWIGLU>(wn, nj) + (lane & 31), chk));
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
        af[buf][mi] = *reinterpret_cast<const bf16x8_t*>(
            As + lds_off(wm * C::WM + mi * 32 + (lane & 31), chk));
    };
    fetch(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) fetch(kk + 1, (kk + 1) & 1);
      // the reads above go out before this sub-step's MFMAs (the scheduler
      // would otherwise reuse their registers and serialize read and multiply)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
        for (int nj = 0; nj < C::NJ; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][mi], bfr[kk & 1][nj],
                                                                acc[mi][nj], 0, 0, 0);
      }
    }
  };

  constexpr int NST = C::NST;
  // loads of the NST - 2 newest steps that may stay in flight at a wait
  constexpr int INFLIGHT = (C::A_LOADS + C::B_LOADS) * (NST - 2);
  static_assert(INFLIGHT <= 63, "vmcnt range");
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  // steps past the end reload the last one (in bounds, never read)
  auto kpos = [&](int k) { return k_begin + (k < nk ? k : nk - 1) * BK; };
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) issue(j, kpos(j));
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(INFLIGHT) : "memory");  // stage 0 has landed
  __syncthreads();
  int st = 0, st_issue = NST - 1;
  for (int k = 0; k < nk; ++k) {
    issue(st_issue, kpos(k + NST - 1));  // the stage read in step k - 1
    compute(st);
    // this wave's part of stage k+1 has landed (later steps' loads may be in
    // flight); the barrier makes every wave's part visible and frees stage k
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(INFLIGHT) : "memory");
    __syncthreads();
    st = st == NST - 1 ? 0 : st + 1;
    st_issue = st_issue == NST - 1 ? 0 : st_issue + 1;
  }
  // the loads of the clamped last steps land before the LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}


// Row (within the tile) of accumulator element r of a 32x32 sub-tile, for
// this lane; the lane's column is lane % 32.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// H = silu(A W1^T) * (A W3^T) per group.
template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void ffn1_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ int gtab[kMaxGroups + 1];
  constexpr int HALF = C::BN / 2;
  static_assert(C::BM * (HALF + 8) <= C::LDS_ELEMS, "the H tile fits in the LDS stages");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_table(gtab, a.tiles1, a.E);
  const int total = gtab[a.E + 1];
  const int nb = gridDim.x;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const i32x4_t rx = a.perm ? rsrc4(a.x, static_cast<uint32_t>(a.T) * row_bytes)
                            : rsrc4(a.xperm, static_cast<uint32_t>(a.TK) * row_bytes);
  const i32x4_t rxs = rsrc4(a.x, static_cast<uint32_t>(a.T) * row_bytes);
  uint16_t* H = static_cast<uint16_t*>(a.H);
  for (int tile = xcd_logical_block(blockIdx.x, nb); tile < total; tile += nb) {
    TileCoord tc = tile_coord(a, gtab, tile, C::BM, a.I, a.Is, HALF);
    tc.g = __builtin_amdgcn_readfirstlane(tc.g);
    tc.rows = __builtin_amdgcn_readfirstlane(tc.rows);
    tc.rbase = __builtin_amdgcn_readfirstlane(tc.rbase);
    tc.m = __builtin_amdgcn_readfirstlane(tc.m);
    tc.n = __builtin_amdgcn_readfirstlane(tc.n);
    const bool shared = tc.g == a.E;
    const int Ig = shared ? a.Is : a.I;
    const int rows_left = tc.rows - tc.m * C::BM;
    uint32_t aoff[C::A_LOADS];
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int r = tc.m * C::BM + r0 + p * C::RPP;
      uint32_t off = kInvalidRow;
      if (r < tc.rows) {
        if (shared) {
          off = static_cast<uint32_t>(r) * row_bytes;
        } else if (a.perm) {
          const int tok = a.perm[tc.rbase + r];
          if (tok >= 0 && tok < a.T) off = static_cast<uint32_t>(tok) * row_bytes;
        } else {
          off = static_cast<uint32_t>(tc.rbase + r) * row_bytes;
        }
      }
      aoff[p] = off;
    }
    const uint16_t* W = shared ? static_cast<const uint16_t*>(a.ws13)
                               : static_cast<const uint16_t*>(a.w13) +
                                     static_cast<int64_t>(tc.g) * 2 * a.I * a.d;
    const i32x4_t rw = rsrc4(W, static_cast<uint32_t>(2 * Ig) * row_bytes);
    uint32_t boff[C::B_LOADS];
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      const bool up = lr >= HALF;
      const int col = tc.n * HALF + (up ? lr - HALF : lr);
      boff[p] = col < Ig ? static_cast<uint32_t>(up ? Ig + col : col) * row_bytes : kInvalidRow;
    }
    f32x16_t acc[C::MI][C::NJ];
    gemm_tile<C, true>(lds, shared ? rxs : rx, aoff, rw, boff, 0, a.d, 0, acc);

    const int64_t hrow0 = (shared ? a.TK : tc.rbase) + static_cast<int64_t>(tc.m) * C::BM;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ / 2; ++nj) {
        const int col = wn * (C::WN / 2) + nj * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float h = silu_f32(acc[mi][nj][r]) * acc[mi][nj + C::NJ / 2][r];
          out_put<C, HALF>(lds, wm * C::WM + mi * 32 + acc_row(lane, r), col, h);
        }
      }
    __syncthreads();
    out_flush<C, HALF>(lds, H + hrow0 * a.ldh + tc.n * HALF, a.ldh, rows_left,
                       Ig - tc.n * HALF);
    __syncthreads();
  }
}

// y = H W2^T per group: routed rows to y_perm, shared rows to y_shared.
template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void ffn2_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ int gtab[kMaxGroups + 1];
  static_assert(C::BM * (C::BN + 8) <= C::LDS_ELEMS, "the output tile fits in the LDS stages");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_table(gtab, a.tiles2, a.E);
  const int total = gtab[a.E + 1];
  const int nb = gridDim.x;
  const uint32_t hrow_bytes = static_cast<uint32_t>(a.ldh) * 2u;
  const int64_t hrows = a.TK + (a.Is > 0 ? a.T : 0);
  const i32x4_t rh = rsrc4(a.H, static_cast<uint32_t>(hrows) * hrow_bytes);
  for (int tile = xcd_logical_block(blockIdx.x, nb); tile < total; tile += nb) {
    TileCoord tc = tile_coord(a, gtab, tile, C::BM, a.d, a.d, C::BN);
    tc.g = __builtin_amdgcn_readfirstlane(tc.g);
    tc.rows = __builtin_amdgcn_readfirstlane(tc.rows);
    tc.rbase = __builtin_amdgcn_readfirstlane(tc.rbase);
    tc.m = __builtin_amdgcn_readfirstlane(tc.m);
    tc.n = __builtin_amdgcn_readfirstlane(tc.n);
    const bool shared = tc.g == a.E;
    const int Ig = shared ? a.Is : a.I;
    const int64_t hrow0 = (shared ? a.TK : tc.rbase) + static_cast<int64_t>(tc.m) * C::BM;
    const int rows_left = tc.rows - tc.m * C::BM;
    uint32_t aoff[C::A_LOADS];
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      aoff[p] = lr < rows_left ? static_cast<uint32_t>(hrow0 + lr) * hrow_bytes : kInvalidRow;
    }
    const uint16_t* W = shared ? static_cast<const uint16_t*>(a.ws2)
                               : static_cast<const uint16_t*>(a.w2) +
                                     static_cast<int64_t>(tc.g) * a.d * a.I;
    const uint32_t wrow_bytes = static_cast<uint32_t>(Ig) * 2u;
    const i32x4_t rw = rsrc4(W, static_cast<uint32_t>(a.d) * wrow_bytes);
    uint32_t boff[C::B_LOADS];
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = tc.n * C::BN + r0 + p * C::RPP;
      boff[p] = row < a.d ? static_cast<uint32_t>(row) * wrow_bytes : kInvalidRow;
    }
    f32x16_t acc[C::MI][C::NJ];
    gemm_tile<C, false>(lds, rh, aoff, rw, boff, 0, Ig, 0, acc);

    uint16_t* out = shared ? static_cast<uint16_t*>(a.yshared) +
                                 static_cast<int64_t>(tc.m) * C::BM * a.d
                           : static_cast<uint16_t*>(a.yperm) +
                                 (static_cast<int64_t>(tc.rbase) + tc.m * C::BM) * a.d;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) {
        const int col = wn * C::WN + nj * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          out_put<C, C::BN>(lds, wm * C::WM + mi * 32 + acc_row(lane, r), col, acc[mi][nj][r]);
      }
    __syncthreads();
    out_flush<C, C::BN>(lds, out + tc.n * C::BN, a.d, rows_left, a.d - tc.n * C::BN);
    __syncthreads();
  }
}

// Router: partial[s][t][e] = sum over k-split s of x[t, k mod d] * wsplit[e, k],
// k in [0, 3d). Grid: (m-tiles * n-tiles, splits).
template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void router_bf16_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wsplit,
                                                               int64_t T, int d, int E, int kchunk,
                                                               float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  const int ntn = (E + C::BN - 1) / C::BN;
  const int64_t m = blockIdx.x / ntn;
  const int n = blockIdx.x % ntn;
  const int split = blockIdx.y;
  const int k_begin = split * kchunk;
  const int k_end = min(3 * d, k_begin + kchunk);
  const uint32_t row_bytes = static_cast<uint32_t>(d) * 2u;
  const i32x4_t rx = rsrc4(x, static_cast<uint32_t>(T) * row_bytes);
  const i32x4_t rw = rsrc4(wsplit, static_cast<uint32_t>(E) * 3u * row_bytes);
  uint32_t aoff[C::A_LOADS];
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) {
    const int64_t t = m * C::BM + r0 + p * C::RPP;
    aoff[p] = t < T ? static_cast<uint32_t>(t) * row_bytes : kInvalidRow;
  }
  uint32_t boff[C::B_LOADS];
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) {
    const int e = n * C::BN + r0 + p * C::RPP;
    boff[p] = e < E ? static_cast<uint32_t>(e) * 3u * row_bytes : kInvalidRow;
  }
  f32x16_t acc[C::MI][C::NJ];
  gemm_tile<C, false>(lds, rx, aoff, rw, boff, k_begin, k_end, d, acc);
  float* out = partial + static_cast<int64_t>(split) * T * E;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) {
      const int e = n * C::BN + wn * C::WN + nj * 32 + (lane & 31);
      if (e >= E) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m * C::BM + wm * C::WM + mi * 32 + acc_row(lane, r);
        if (t < T) out[t * E + e] = acc[mi][nj][r];
      }
    }
}

// wsplit[e, j*d + k] = j-th bf16 term of w[e, k]: hi = bf16(w),
// mid = bf16(w - hi), lo = bf16(w - hi - mid). Each subtraction is exact, and
// three 8-bit terms cover the 24-bit fp32 significand, so hi + mid + lo == w.
__global__ __launch_bounds__(256) void split_router_kernel(const float* __restrict__ w, int64_t E,
                                                           int d, uint16_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= E * d) return;
  const int64_t e = i / d;
  const int k = static_cast<int>(i % d);
  const float v = w[i];
  const uint16_t hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  const uint16_t lo = f32_to_bf16(r2);
  uint16_t* row = out + e * 3 * d;
  row[k] = hi;
  row[d + k] = mid;
  row[2 * d + k] = lo;
}

template <class K>
int occupancy_blocks(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

template <class C1, class C2>
hipError_t launch_ffn_bf16_cfg(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  static int occ1 = 0, occ2 = 0;
  if (!occ1) occ1 = occupancy_blocks(ffn1_bf16_kernel<C1>, C1::NT);
  if (!occ2) occ2 = occupancy_blocks(ffn2_bf16_kernel<C2>, C2::NT);
  const int cus = device_cu_count();
  // persistent grids, multiples of 8 for the XCD remap
  const int g1 = ((cus * occ1 + 7) / 8) * 8;
  const int g2 = ((cus * occ2 + 7) / 8) * 8;
  hipLaunchKernelGGL((ffn1_bf16_kernel<C1>), dim3(g1), dim3(C1::NT), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;
  hipLaunchKernelGGL((ffn2_bf16_kernel<C2>), dim3(g2), dim3(C2::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

GemmTiling choose_tiling(int64_t T, int K, int E, int w_dtype) {
  GemmTiling t{};
  const double rows_per_expert = static_cast<double>(T) * K / E;
  if (w_dtype == 2) return choose_tiling_fp8(rows_per_expert);
  if (rows_per_expert < 48.0) {
    t.bm1 = TileDecode::BM; t.bnh1 = TileDecode::BN / 2;
    t.bm2 = TileDecode::BM; t.bn2 = TileDecode::BN; t.variant = 1;
  } else {
    t.bm1 = TilePrefill::BM; t.bnh1 = TilePrefill::BN / 2;
    t.bm2 = TilePrefill::BM; t.bn2 = TilePrefill::BN; t.variant = 0;
  }
  return t;
}

hipError_t launch_ffn_bf16(const FfnArgs& a, const GemmTiling& t, hipStream_t s, hipEvent_t mid) {
  if (t.variant == 1) return launch_ffn_bf16_cfg<TileDecode, TileDecode>(a, s, mid);
  return launch_ffn_bf16_cfg<TilePrefill, TilePrefill>(a, s, mid);
}

int router_splits(int64_t T, int d, int E, int act_dtype) {
  if (act_dtype != 1) return 1;
  // enough workgroups to cover the chip; each split a multiple of 64 in k
  const int64_t base = ((T + 127) / 128) * ((E + 127) / 128);
  const int cus = device_cu_count();
  int s = 1;
  while (base * s < 2 * cus && (3 * d) / (64 * (s * 2)) >= 4) s *= 2;
  return s;
}

size_t router_split_bytes(int d, int E) { return static_cast<size_t>(E) * 3 * d * 2; }

hipError_t launch_router_logits_bf16(const void* x, const float* w_router, int64_t T, int d, int E,
                                     int splits, uint16_t* wsplit, float* partial, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t n = static_cast<int64_t>(E) * d;
  hipLaunchKernelGGL(split_router_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, w_router, static_cast<int64_t>(E), d, wsplit);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int K3 = 3 * d;
  int kchunk = ((K3 / splits + 63) / 64) * 64;
  using C = TilePrefill;
  const int64_t mt = (T + C::BM - 1) / C::BM;
  const int ntn = (E + C::BN - 1) / C::BN;
  hipLaunchKernelGGL(router_bf16_kernel<C>, dim3(static_cast<unsigned>(mt * ntn), splits),
                     dim3(C::NT), 0, s, static_cast<const uint16_t*>(x), wsplit, T, d, E, kchunk,
                     partial);
  return hipGetLastError();
}

}  // namespace dsmoe
