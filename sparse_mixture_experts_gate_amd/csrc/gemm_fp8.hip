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
#include "gemm_fp8_core.h"

namespace dsmoe {

namespace {

using T8Gate = Tile8<128, 256, 64, 64>;        // 8 waves, H tile 128 x 128, 144 KB ring
using T8Down = Tile8<128, 256, 64, 64>;        // 8 waves, 144 KB ring
using T8GateDec = Tile8<32, 256, 32, 64, 4, true>;   // 4 waves, 144 KB ring
using T8DownDec = Tile8<32, 128, 32, 64, 6, true>;   // 2 waves, 120 KB ring


// H (E4M3 + 1x128 scales) = quant(silu(A W1^T) * (A W3^T)); tile = 128 H
// columns. Routed rows of A are gathered through perm: the token indices of a
// tile's rows come into an LDS slot by the same asynchronous loads as the
// operands, one tile ahead, so that the tile loop issues no compiler-visible
// global loads.
// TRAIN also stores, for the backward, the pre-activations a = x W1^T and
// b = x W3^T (bf16, row r of a.gu: a in columns [0, Ig), b in [Ig, 2 Ig), row
// stride 2 ldh) and H in bf16 (a.h16 [rows, ldh]).
template <class C, bool TRAIN>
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
  const i32x4_t rxs = rsrc4(a.x, static_cast<uint32_t>(a.T) * static_cast<uint32_t>(a.d));
  const i32x4_t rx =
      a.perm ? rxs : rsrc4(a.xperm, static_cast<uint32_t>(a.TK) * static_cast<uint32_t>(a.d));
  // activation scales, k-block major (scale_rows_kernel): the routed rows in
  // the permuted order, then the shared rows
  const int64_t srows = a.TK + (a.Is > 0 ? a.T : 0);
  const i32x4_t rsx =
      rsrc4(a.xsT, static_cast<uint32_t>(srows) * static_cast<uint32_t>(dkb) * 4u);
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
    if (tid < C::BM && src_row(tid) >= 0) {
      const int gr = c.m * C::BM + tid;
      op.sa_off = static_cast<uint32_t>(c.shared ? a.TK + gr : c.rbase + gr) * 4u;
    }
    op.sa_step = static_cast<uint32_t>(srows) * 4u;
    op.ra = c.shared ? rxs : rx;
    op.rsa = rsx;
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
    // every wave of the tile needs the same two block scales: wave 0 loads them
    op.sb_lo = wave == 0 ? static_cast<uint32_t>(c.n * dkb) * 4u : kInvalidRow;
    op.sb_hi = wave == 0 ? static_cast<uint32_t>((Ig / 128 + c.n) * dkb) * 4u : kInvalidRow;
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
        a.H_scale[c.n * srows + hrow0 + lr] = amax == 0.0f ? 1.0f : amax / 448.0f;
      if constexpr (TRAIN) {
        const int Ig = c.shared ? a.Is : a.I;
        const int64_t hr = hrow0 + lr;
        const int col0 = c.n * HALF + wn * (C::WN / 2) + 4 * (lane >> 5);
        uint16_t* gp = static_cast<uint16_t*>(a.gu) + hr * 2 * a.ldh;
        uint16_t* h16 = static_cast<uint16_t*>(a.h16) + hr * a.ldh;
#pragma unroll
        for (int nj = 0; nj < NJH; ++nj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = col0 + nj * 32 + 8 * g;
            const f32x16_t& gv = acc[mi][nj];
            const f32x16_t& uv = acc[mi][nj + NJH];
            const float* v = &h[mi][nj][4 * g];
            *reinterpret_cast<uint2*>(gp + col) =
                pack_bf16x4(gv[4 * g], gv[4 * g + 1], gv[4 * g + 2], gv[4 * g + 3]);
            *reinterpret_cast<uint2*>(gp + Ig + col) =
                pack_bf16x4(uv[4 * g], uv[4 * g + 1], uv[4 * g + 2], uv[4 * g + 3]);
            *reinterpret_cast<uint2*>(h16 + col) = pack_bf16x4(v[0], v[1], v[2], v[3]);
          }
      }
    }
    // red[] is rewritten by the next tile's epilogue only after at least one
    // more k block, whose barrier orders these reads first
  };
  gemm8_stream<C, true>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of, epilogue, 0);
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
  // the wave (row 0 of the wave grid) that loads this wave's weight block scale
  const int sbw = (wn / (128 / C::WN)) * (128 / C::WN);
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles2, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const int hkb = a.ldh / 128;
  const int64_t hrows = a.TK + (a.Is > 0 ? a.T : 0);
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
    // H codes through a resource based at the tile's first row (64-bit base,
    // 32-bit offsets inside the tile), so H itself may exceed 2^31 bytes
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left ? static_cast<uint32_t>(lr) * static_cast<uint32_t>(a.ldh)
                                : kInvalidRow;
    }
    op.ra = rsrc4(static_cast<const uint8_t*>(a.H) + hrow0 * a.ldh,
                  static_cast<uint32_t>(rows_left < C::BM ? rows_left : C::BM) *
                      static_cast<uint32_t>(a.ldh));
    op.sa_off = (tid < C::BM && tid < rows_left) ? static_cast<uint32_t>(hrow0 + tid) * 4u
                                                 : kInvalidRow;
    op.sa_step = static_cast<uint32_t>(hrows) * 4u;
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
    // the first wave of each 128-column scale block loads its block scale
    op.sb_lo = op.sb_hi =
        wave == sbw ? static_cast<uint32_t>(((c.n * C::BN + wn * C::WN) / 128) * ikb) * 4u
                    : kInvalidRow;
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
  gemm8_stream<C, false>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of, epilogue, sbw);
}

template <class K>
int occupancy8(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

// The activation scales in the layout the gate/up GEMM reads: k-block major,
// the routed rows in the permuted order (each from its token's row of
// x_scale, or from the scales of x_perm), then the shared rows, so that a
// tile's row scales of one k block are one contiguous run of 4-byte values
// instead of one cache line per row.
__global__ __launch_bounds__(256) void scale_rows_kernel(FfnArgs a, int dkb, int64_t srows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= srows * dkb) return;
  const int kb = static_cast<int>(i / srows);
  const int64_t r = i - kb * srows;
  float v = 0.0f;
  if (r < a.TK) {
    if (a.perm) {
      const int tok = a.perm[r];
      if (tok >= 0 && tok < a.T) v = a.x_scale[static_cast<int64_t>(tok) * dkb + kb];
    } else {
      v = a.xperm_scale[r * dkb + kb];
    }
  } else {
    v = a.x_scale[(r - a.TK) * dkb + kb];
  }
  a.xsT[i] = v;
}

template <class C1, class C2, bool TRAIN>
hipError_t launch_fp8_pair(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  static int occ1 = 0, occ2 = 0;
  if (!occ1) occ1 = occupancy8(ffn1_fp8_kernel<C1, TRAIN>, C1::NT);
  if (!occ2) occ2 = occupancy8(ffn2_fp8_kernel<C2>, C2::NT);
  const int cus = device_cu_count();
  const int g1 = ((cus * occ1 + 7) / 8) * 8;
  const int g2 = ((cus * occ2 + 7) / 8) * 8;
  const int dkb = a.d / 128;
  const int64_t srows = a.TK + (a.Is > 0 ? a.T : 0);
  if (srows > 0) {
    hipLaunchKernelGGL(scale_rows_kernel, dim3(static_cast<unsigned>((srows * dkb + 255) / 256)),
                       dim3(256), 0, s, a, dkb, srows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ffn1_fp8_kernel<C1, TRAIN>), dim3(g1), dim3(C1::NT), 0, s, a);
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
  if (a.gu) {
    if (t.variant == 1) return launch_fp8_pair<T8GateDec, T8DownDec, true>(a, s, mid);
    return launch_fp8_pair<T8Gate, T8Down, true>(a, s, mid);
  }
  if (t.variant == 1) return launch_fp8_pair<T8GateDec, T8DownDec, false>(a, s, mid);
  return launch_fp8_pair<T8Gate, T8Down, false>(a, s, mid);
}

}  // namespace dsmoe
