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
#include "gemm_bf16_core.h"

namespace dsmoe {

namespace {

// acc += one 64-wide k-step of the tile in ring stage st. Within the step the
// LDS fragments of the next 16-wide sub-step are read while the current one
// multiplies. SWAP puts the B (weight) fragment first, so that acc holds the
// transposed tile: lane l then owns output row l % 32 and, per group of four
// registers, four adjacent output columns (one 8-byte bf16 store).
template <class C, bool SWIGLU, bool SWAP>
__device__ __forceinline__ void stage_mma(const uint16_t* lds, int st, int wm, int wn, int lane,
                                          f32x16_t (&acc)[C::MI][C::NJ]) {
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
      for (int nj = 0; nj < C::NJ; ++nj) {
        if constexpr (SWAP)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][nj], af[kk & 1][mi],
                                                                acc[mi][nj], 0, 0, 0);
        else
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][mi], bfr[kk & 1][nj],
                                                                acc[mi][nj], 0, 0, 0);
      }
    }
  }
}

// acc = A * B^T over k in [k_begin, k_end) (multiples of 64) for one tile.
// Operands come from buffers (ra, rb) through a 32-bit byte offset per thread
// and row (the k = 0 element of the row); offsets at or beyond the buffer
// size (kInvalidRow) read as zeros, so padding rows cost no branches. With
// a_kmod != 0 the A column is k mod a_kmod (router: the same activations meet
// the three weight terms). Loads run NST - 1 k-steps ahead through the ring,
// one barrier per step.
template <class C, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(uint16_t* lds, i32x4_t ra,
                                          const uint32_t (&aoff)[C::A_LOADS], i32x4_t rb,
                                          const uint32_t (&boff)[C::B_LOADS], int k_begin,
                                          int k_end, int a_kmod, f32x16_t (&acc)[C::MI][C::NJ]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  zero_acc<C>(acc);
  uint32_t ao[C::A_LOADS], bo[C::B_LOADS];
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) ao[p] = aoff[p];
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) bo[p] = boff[p];
  swizzle_rows<C>(ao);
  swizzle_rows<C>(bo);
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int st, int k0) {
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
    const uint32_t ka = a_kmod ? static_cast<uint32_t>(k0 % a_kmod) * 2u : kb;
    stage_issue<C>(lds0, st, wave, ra, ao, ka, rb, bo, kb);
  };
  constexpr int NST = C::NST;
  constexpr int INFLIGHT = kInflight<C>;
  static_assert(INFLIGHT <= 63, "vmcnt range");
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  // steps past the end reload the last one (in bounds, never read)
  auto kpos = [&](int k) { return k_begin + (k < nk ? k : nk - 1) * BK; };
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) issue(j, kpos(j));
  vm_wait<INFLIGHT>();  // stage 0 has landed
  __syncthreads();
  int st = 0, st_issue = NST - 1;
  for (int k = 0; k < nk; ++k) {
    issue(st_issue, kpos(k + NST - 1));  // the stage read in step k - 1
    stage_mma<C, SWIGLU, false>(lds, st, wm, wn, lane, acc);
    // this wave's part of stage k+1 has landed (later steps' loads may be in
    // flight); the barrier makes every wave's part visible and frees stage k
    vm_wait<INFLIGHT>();
    __syncthreads();
    st = st == NST - 1 ? 0 : st + 1;
    st_issue = st_issue == NST - 1 ? 0 : st_issue + 1;
  }
  // the loads of the clamped last steps land before the LDS is reused
  vm_wait<0>();
  __syncthreads();
}


// H = silu(A W1^T) * (A W3^T) per group. Routed rows of A are gathered
// through perm: the token indices of a tile are brought into an LDS slot by
// the same asynchronous loads as the operands, one tile ahead, so that the
// tile loop issues no compiler-visible global loads. TRAIN also stores the
// pre-activations (bf16) for the backward: row r of a.gu holds A W1^T in
// columns [0, Ig) and A W3^T in [Ig, 2 Ig), row stride 2 ldh.
template <class C, bool TRAIN>
__global__ __launch_bounds__(C::NT, C::MINW) void ffn1_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ GroupTables gt;
  constexpr int PS = C::BM > 64 ? C::BM : 64;  // one dma4 per 64 rows
  __shared__ __attribute__((aligned(16))) int pslot[2][PS];
  constexpr int HALF = C::BN / 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles1, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const i32x4_t rxs = rsrc4(a.x, static_cast<uint32_t>(a.T) * row_bytes);
  const i32x4_t rx = a.perm ? rxs : rsrc4(a.xperm, static_cast<uint32_t>(a.TK) * row_bytes);
  const i32x4_t rperm = rsrc4(a.perm, static_cast<uint32_t>(a.TK) * 4u);
  const int nk = a.d / BK;
  uint16_t* H = static_cast<uint16_t*>(a.H);

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
  // the first tile's indices, and the second's one tile ahead
  fetch_perm(first, 0);
  if (first + nb < total) fetch_perm(first + nb, 1);
  vm_wait<0>();
  lds_barrier();

  auto next_ops = [&](int tile, int index, StreamOps<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int* slot = pslot[index & 1];
    if (index > 0) {
      // slot index & 1 was filled while tile index - 1 was issued, nk steps
      // ago: landed once NST - 2 further steps of loads were issued after it
      if (nk < C::NST - 1) {
        vm_wait<0>();
        lds_barrier();
      }
      if (tile + nb < total) fetch_perm(tile + nb, (index + 1) & 1);
    }
    const int Ig = c.shared ? a.Is : a.I;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int r = c.m * C::BM + r0 + p * C::RPP;
      uint32_t off = kInvalidRow;
      if (r < c.rows) {
        if (c.shared) {
          off = static_cast<uint32_t>(r) * row_bytes;
        } else if (a.perm) {
          const int tok = slot[r0 + p * C::RPP];
          if (tok >= 0 && tok < a.T) off = static_cast<uint32_t>(tok) * row_bytes;
        } else {
          off = static_cast<uint32_t>(c.rbase + r) * row_bytes;
        }
      }
      op.ao[p] = off;
    }
    op.ra = c.shared ? rxs : rx;
    const uint16_t* W = c.shared ? static_cast<const uint16_t*>(a.ws13)
                                 : static_cast<const uint16_t*>(a.w13) +
                                       static_cast<int64_t>(c.g) * 2 * a.I * a.d;
    op.rb = rsrc4(W, static_cast<uint32_t>(2 * Ig) * row_bytes);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      const bool up = lr >= HALF;
      const int col = c.n * HALF + (up ? lr - HALF : lr);
      op.bo[p] = col < Ig ? static_cast<uint32_t>(up ? Ig + col : col) * row_bytes : kInvalidRow;
    }
    swizzle_rows<C>(op.ao);
    swizzle_rows<C>(op.bo);
    op.nk = nk;
  };
  auto nk_of = [&](int) { return nk; };
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int rows_left = c.rows - c.m * C::BM;
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int row = wm * C::WM + mi * 32 + (lane & 31);
      if (row >= rows_left) continue;
      uint16_t* hp = H + (hrow0 + row) * a.ldh;
#pragma unroll
      for (int nj = 0; nj < C::NJ / 2; ++nj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = c.n * HALF + wn * (C::WN / 2) + nj * 32 + 8 * g + 4 * (lane >> 5);
          if (col >= Ig) continue;
          const f32x16_t& gv = acc[mi][nj];
          const f32x16_t& uv = acc[mi][nj + C::NJ / 2];
          *reinterpret_cast<uint2*>(hp + col) =
              pack_bf16x4(silu_f32(gv[4 * g]) * uv[4 * g], silu_f32(gv[4 * g + 1]) * uv[4 * g + 1],
                          silu_f32(gv[4 * g + 2]) * uv[4 * g + 2],
                          silu_f32(gv[4 * g + 3]) * uv[4 * g + 3]);
          if constexpr (TRAIN) {
            uint16_t* gp = static_cast<uint16_t*>(a.gu) + (hrow0 + row) * 2 * a.ldh + col;
            *reinterpret_cast<uint2*>(gp) =
                pack_bf16x4(gv[4 * g], gv[4 * g + 1], gv[4 * g + 2], gv[4 * g + 3]);
            *reinterpret_cast<uint2*>(gp + Ig) =
                pack_bf16x4(uv[4 * g], uv[4 * g + 1], uv[4 * g + 2], uv[4 * g + 3]);
          }
        }
    }
  };
  auto rows_of = [&](int tile) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    return c.rows - c.m * C::BM;
  };
  gemm_stream<C, true, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, true, -1,
              false, false, decltype(rows_of)>(lds, first, nb, total, next_ops, nk_of, epilogue,
                                               rows_of);
}

// y = H W2^T per group: routed rows to y_perm, shared rows to y_shared.
template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void ffn2_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
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
  const uint32_t hrow_bytes = static_cast<uint32_t>(a.ldh) * 2u;
  // the shared group's tiles are the last ones
  const int shared_first = a.E > 0 ? gt.gnext[a.E - 1] : 0;

  auto next_ops = [&](int tile, int, StreamOps<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    const int rows_left = c.rows - c.m * C::BM;
    // H through a resource based at the tile's first row (64-bit base, 32-bit
    // offsets inside the tile), so H itself may exceed 2^31 bytes
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left ? static_cast<uint32_t>(lr) * hrow_bytes : kInvalidRow;
    }
    op.ra = rsrc4(static_cast<const uint16_t*>(a.H) + hrow0 * a.ldh,
                  static_cast<uint32_t>(rows_left < C::BM ? rows_left : C::BM) * hrow_bytes);
    const uint16_t* W = c.shared ? static_cast<const uint16_t*>(a.ws2)
                                 : static_cast<const uint16_t*>(a.w2) +
                                       static_cast<int64_t>(c.g) * a.d * a.I;
    const uint32_t wrow_bytes = static_cast<uint32_t>(Ig) * 2u;
    op.rb = rsrc4(W, static_cast<uint32_t>(a.d) * wrow_bytes);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = c.n * C::BN + r0 + p * C::RPP;
      op.bo[p] = row < a.d ? static_cast<uint32_t>(row) * wrow_bytes : kInvalidRow;
    }
    swizzle_rows<C>(op.ao);
    swizzle_rows<C>(op.bo);
    op.nk = Ig / BK;
  };
  auto nk_of = [&](int tile) { return (tile >= shared_first ? a.Is : a.I) / BK; };
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
          *reinterpret_cast<uint2*>(yp + col) =
              pack_bf16x4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
        }
    }
  };
  auto rows_of = [&](int tile) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    return c.rows - c.m * C::BM;
  };
  gemm_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, true, -1,
              false, false, decltype(rows_of)>(lds, first, nb, total, next_ops, nk_of, epilogue,
                                               rows_of);
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

template <class C1, class C2, bool TRAIN>
hipError_t launch_ffn_bf16_cfg(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  static int occ1 = 0, occ2 = 0;
  if (!occ1) occ1 = occupancy_blocks(ffn1_bf16_kernel<C1, TRAIN>, C1::NT);
  if (!occ2) occ2 = occupancy_blocks(ffn2_bf16_kernel<C2>, C2::NT);
  const int cus = device_cu_count();
  // persistent grids, multiples of 8 for the XCD remap
  const int g1 = ((cus * occ1 + 7) / 8) * 8;
  const int g2 = ((cus * occ2 + 7) / 8) * 8;
  hipLaunchKernelGGL((ffn1_bf16_kernel<C1, TRAIN>), dim3(g1), dim3(C1::NT), 0, s, a);
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
  if (w_dtype == 0) return tiling_f32();
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
  if (a.gu) {
    if (t.variant == 1) return launch_ffn_bf16_cfg<TileDecode, TileDecode, true>(a, s, mid);
    return launch_ffn_bf16_cfg<TilePrefill, TilePrefill, true>(a, s, mid);
  }
  if (t.variant == 1) return launch_ffn_bf16_cfg<TileDecode, TileDecode, false>(a, s, mid);
  return launch_ffn_bf16_cfg<TilePrefill, TilePrefill, false>(a, s, mid);
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
