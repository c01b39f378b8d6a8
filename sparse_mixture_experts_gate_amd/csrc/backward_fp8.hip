// FP8 backward of the layer on gfx950: the forward pass computes in E4M3, the
// backward in E5M2 (10100.com DeepSeek-V3 technical-report article, FP8
// paragraph), with the fine-grained scaling of mhpq.cn "DeepSeek-V3
// 高效训练关键技术全景解析" §4.1: activations and gradients in 1x128 groups,
// weights in 128x128 blocks, fp32 accumulation. Every GEMM of the backward
// contracts FP8 operands quantized along its own contraction axis:
//   - input gradients (contraction over a projection's output channels):
//       dH   = E5M2(dY, 1x128 along d) . W2      -> SwiGLU backward -> [da | db]
//       dA   = E5M2([da | db], 1x128 along 2I) . [W1; W3]
//     with the forward's E4M3 weight blocks, read from transposed copies
//     (W2^T [I, d], [W1; W3]^T [d, 2I]) so that both operands run along the
//     contraction; a 128x128 block of W is a block of W^T, scale and all;
//   - weight gradients (contraction over an expert's tokens):
//       dW2  = E5M2(dY)^T E4M3(H),  dW13 = E5M2([da | db])^T E4M3(x)
//     with both operands in 128x1 tiles, i.e. 128 consecutive rows of the
//     expert's segment per scale and channel; a quantizer writes them
//     transposed ([channels, tokens] per expert) so the GEMM reads both
//     operands along the contraction as well.
// The GEMMs run on the FP8 k-stream core (gemm_fp8_core.h) with the formats
// set per operand; the weight-gradient product has a scale per row and 128
// tokens on both sides, so each accumulated value gets its own product of
// the two scales.
#pragma clang fp contract(off)

#include "device_common.h"
#include "internal.h"
#include "tile_schedule.h"
#include "gemm_fp8_core.h"

namespace dsmoe {

namespace {

constexpr int kE4M3 = 0, kE5M2 = 1;

using T8Bwd = Tile8<128, 256, 64, 64>;  // 8 waves of 64 x 64, 144 KB ring

template <class K>
int occupancy_fp8b(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

__device__ __forceinline__ float silu_grad(float a, float s) { return s * (1.0f + a * (1.0f - s)); }

__device__ __forceinline__ float sigmoid_fast(float a) { return 1.0f / (1.0f + __expf(-a)); }

// ---- dH = E5M2(dY) W2 with the SwiGLU backward epilogue --------------------
//
// Per group (routed expert or the shared expert): rows of the E5M2 gradient
// (1x128 scales along d) times the rows of W2^T (I rows of d codes, 128x128
// block scales). Tiles of 128 rows x 256 intermediate columns; the epilogue
// reads the saved pre-activations a, b (bf16), forms da = dH b silu'(a) and
// db = dH silu(a), writes them in bf16 (for the weight-gradient quantizer)
// and as E5M2 codes with 1x128 scales along [da | db] (each 128 columns of
// the tile are one group, spread over two waves).
template <class C>
__global__ __launch_bounds__(C::NT, 2) void dgrad2_fp8_kernel(BwdFp8Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_sa[C::NST * C::NT];
  __shared__ __attribute__((aligned(16))) float lds_sb[C::NST * C::NWAVES * 2];
  __shared__ float red[2][C::WAVES_N][C::BM];
  __shared__ GroupTables gt;
  static_assert(128 % C::WN == 0 && C::BN % 128 == 0, "128-column groups of whole waves");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // the wave (row 0 of the wave grid) that loads this wave's weight block scale
  const int sbw = (wn / (128 / C::WN)) * (128 / C::WN);
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles_h, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const int dkb = a.d / 128;
  // rows of [da | db] (routed, then shared): the stride of its k-block-major scales
  const int64_t hrows = a.TK + (a.Is > 0 ? a.T : 0);
  const uint32_t d = static_cast<uint32_t>(a.d);
  const i32x4_t rsyr = rsrc4(a.dys, static_cast<uint32_t>(a.TK) * dkb * 4u);
  const i32x4_t rsys = rsrc4(a.dyss, static_cast<uint32_t>(a.T) * dkb * 4u);
  const int nk = a.d / BK8;

  auto next_ops = [&](int tile, int, StreamOps8<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int rows_left = c.rows - c.m * C::BM;
    const int64_t row0 = (c.shared ? 0 : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    // the tile's gradient codes through a resource based at its first row
    // (64-bit base, 32-bit offsets inside the tile)
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left ? static_cast<uint32_t>(lr) * d : kInvalidRow;
    }
    op.sa_off = (tid < C::BM && tid < rows_left) ? static_cast<uint32_t>(row0 + tid) * 4u
                                                 : kInvalidRow;
    op.sa_step = static_cast<uint32_t>(c.shared ? a.T : a.TK) * 4u;  // k-block-major scales
    op.ra = rsrc4((c.shared ? a.dysq : a.dyq) + row0 * a.d,
                  static_cast<uint32_t>(rows_left < C::BM ? rows_left : C::BM) * d);
    op.rsa = c.shared ? rsys : rsyr;
    const uint8_t* W = c.shared ? a.ws2t : a.w2t + static_cast<int64_t>(c.g) * a.I * a.d;
    const float* WS = c.shared ? a.ws2t_scale
                               : a.w2t_scale + static_cast<int64_t>(c.g) * (a.I / 128) * dkb;
    op.rb = rsrc4(W, static_cast<uint32_t>(Ig) * d);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = c.n * C::BN + r0 + p * C::RPP;
      op.bo[p] = row < Ig ? static_cast<uint32_t>(row) * d : kInvalidRow;
    }
    op.rsb = rsrc4(WS, static_cast<uint32_t>(Ig / 128) * dkb * 4u);
    op.sb_lo = op.sb_hi =
        wave == sbw ? static_cast<uint32_t>(((c.n * C::BN + wn * C::WN) / 128) * dkb) * 4u
                    : kInvalidRow;
    swizzle_rows8<C>(op.ao);
    swizzle_rows8<C>(op.bo);
    op.nk = nk;
  };
  auto nk_of = [&](int) { return nk; };
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int rows_left = c.rows - c.m * C::BM;
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    const int col_w = c.n * C::BN + wn * C::WN + 4 * (lane >> 5);  // + 32 nj + 8 g + q
    // da, db of this lane's 16 values per product; row max-abs per wave
    float da[C::MI][C::NJ][16], db[C::MI][C::NJ][16];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int lr = wm * C::WM + mi * 32 + (lane & 31);
      const bool row_ok = lr < rows_left;
      const uint16_t* gp = a.gu + (hrow0 + lr) * 2 * a.ldh;
      float ma = 0.0f, mb = 0.0f;
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = col_w + nj * 32 + 8 * g;
          uint2 av = make_uint2(0u, 0u), bv = make_uint2(0u, 0u);
          if (row_ok && col < Ig) {
            av = *reinterpret_cast<const uint2*>(gp + col);
            bv = *reinterpret_cast<const uint2*>(gp + Ig + col);
          }
          const uint32_t aw[2] = {av.x, av.y}, bw[2] = {bv.x, bv.y};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x = __uint_as_float(q & 1 ? aw[q >> 1] & 0xFFFF0000u : aw[q >> 1] << 16);
            const float y = __uint_as_float(q & 1 ? bw[q >> 1] & 0xFFFF0000u : bw[q >> 1] << 16);
            const float dh = acc[mi][nj][4 * g + q];
            const float s = sigmoid_fast(x);
            const float va = dh * y * silu_grad(x, s);
            const float vb = dh * x * s;
            da[mi][nj][4 * g + q] = va;
            db[mi][nj][4 * g + q] = vb;
            ma = fmaxf(ma, fabsf(va));
            mb = fmaxf(mb, fabsf(vb));
          }
        }
      ma = fmaxf(ma, __shfl_xor(ma, 32, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      if (lane < 32) {
        red[0][wn][wm * C::WM + mi * 32 + lane] = ma;
        red[1][wn][wm * C::WM + mi * 32 + lane] = mb;
      }
    }
    lds_barrier();
    constexpr int WPG = 128 / C::WN;  // waves per 128-column group
    const int w0 = (wn / WPG) * WPG;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int lr = wm * C::WM + mi * 32 + (lane & 31);
      float amax[2] = {0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < WPG; ++w) {
        amax[0] = fmaxf(amax[0], red[0][w0 + w][lr]);
        amax[1] = fmaxf(amax[1], red[1][w0 + w][lr]);
      }
      if (lr >= rows_left) continue;
      const int64_t hrow = hrow0 + lr;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float am = amax[h];
        const float inv = am == 0.0f ? 0.0f : 57344.0f / am;
        const int cbase = h ? Ig : 0;
        uint8_t* qp = a.dgq + hrow * 2 * a.ldh + cbase;
        uint16_t* bp = a.dg + hrow * 2 * a.ldh + cbase;
#pragma unroll
        for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = col_w + nj * 32 + 8 * g;
            if (col >= Ig) continue;
            const float* v = h ? &db[mi][nj][4 * g] : &da[mi][nj][4 * g];
            *reinterpret_cast<uint32_t*>(qp + col) =
                am == 0.0f ? 0u : e5m2_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            *reinterpret_cast<uint2*>(bp + col) = pack_bf16x4(v[0], v[1], v[2], v[3]);
          }
        const int cgrp = c.n * C::BN + w0 * C::WN;  // first column of the wave pair's group
        if (wn == w0 && lane < 32 && cgrp < Ig)
          a.dgs[static_cast<int64_t>((cbase + cgrp) / 128) * hrows + hrow] =
              am == 0.0f ? 1.0f : am / 57344.0f;
      }
    }
    // red[] is rewritten by the next tile's epilogue only after at least one
    // more k block, whose barrier orders these reads first
  };
  gemm8_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, kE4M3,
               kE5M2>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of, epilogue, sbw);
}

// ---- dA = E5M2([da | db]) [W1; W3] --------------------------------------------
//
// Per group: rows of the E5M2 [da | db] (1x128 scales along 2 Ig) times the
// rows of [W1; W3]^T (d rows of 2 Ig codes, 128x128 block scales); bf16 out.
template <class C>
__global__ __launch_bounds__(C::NT, 2) void dgrad1_fp8_kernel(BwdFp8Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_sa[C::NST * C::NT];
  __shared__ __attribute__((aligned(16))) float lds_sb[C::NST * C::NWAVES * 2];
  __shared__ GroupTables gt;
  static_assert(128 % C::WN == 0, "a wave's columns lie in one scale block");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // the wave (row 0 of the wave grid) that loads this wave's weight block scale
  const int sbw = (wn / (128 / C::WN)) * (128 / C::WN);
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles_d, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const int gkb = 2 * a.ldh / 128;
  const uint32_t lrow = 2u * static_cast<uint32_t>(a.ldh);
  const int64_t hrows = a.TK + (a.Is > 0 ? a.T : 0);
  const i32x4_t rsg = rsrc4(a.dgs, static_cast<uint32_t>(hrows) * gkb * 4u);
  const int shared_first = a.E > 0 ? gt.gnext[a.E - 1] : 0;

  auto next_ops = [&](int tile, int, StreamOps8<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int rows_left = c.rows - c.m * C::BM;
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    // the tile's [da | db] codes through a resource based at its first row
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left ? static_cast<uint32_t>(lr) * lrow : kInvalidRow;
    }
    op.sa_off = (tid < C::BM && tid < rows_left) ? static_cast<uint32_t>(hrow0 + tid) * 4u
                                                 : kInvalidRow;
    op.sa_step = static_cast<uint32_t>(hrows) * 4u;  // k-block-major scales
    op.ra = rsrc4(a.dgq + hrow0 * lrow,
                  static_cast<uint32_t>(rows_left < C::BM ? rows_left : C::BM) * lrow);
    op.rsa = rsg;
    const int kb = 2 * Ig / 128;
    const uint8_t* W = c.shared ? a.ws13t : a.w13t + static_cast<int64_t>(c.g) * a.d * 2 * a.I;
    const float* WS = c.shared ? a.ws13t_scale
                               : a.w13t_scale + static_cast<int64_t>(c.g) * (a.d / 128) *
                                                    (2 * a.I / 128);
    op.rb = rsrc4(W, static_cast<uint32_t>(a.d) * 2u * static_cast<uint32_t>(Ig));
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = c.n * C::BN + r0 + p * C::RPP;
      op.bo[p] = row < a.d ? static_cast<uint32_t>(row) * 2u * static_cast<uint32_t>(Ig)
                           : kInvalidRow;
    }
    op.rsb = rsrc4(WS, static_cast<uint32_t>(a.d / 128) * kb * 4u);
    op.sb_lo = op.sb_hi =
        wave == sbw ? static_cast<uint32_t>(((c.n * C::BN + wn * C::WN) / 128) * kb) * 4u
                    : kInvalidRow;
    swizzle_rows8<C>(op.ao);
    swizzle_rows8<C>(op.bo);
    op.nk = kb;
  };
  auto nk_of = [&](int tile) { return 2 * (tile >= shared_first ? a.Is : a.I) / BK8; };
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int rows_left = c.rows - c.m * C::BM;
    uint16_t* out = c.shared ? a.das + static_cast<int64_t>(c.m) * C::BM * a.d
                             : a.dap + (static_cast<int64_t>(c.rbase) + c.m * C::BM) * a.d;
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
  gemm8_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, kE4M3,
               kE5M2>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of, epilogue, sbw);
}

// ---- weight gradients: out_g = A_g B_g^T over the group's tokens ------------
//
// A_g [M, npad_g], B_g [N, npad_g]: transposed 128x1-tile codes (rows are
// channels, contiguous along the group's tokens, padded to a multiple of
// 128 with zeros), scales [rows, npad_g / 128]. Groups: the E routed
// experts, then the shared expert (its own M, N). A group with no token
// reads one block of zeros and stores exact zeros. Tiles: 128 x 256 of the
// output, n fastest inside a group; out fp32, row-major [M, N].
template <class C, int FA, int FB>
__global__ __launch_bounds__(C::NT, 2) void wgrad_fp8_kernel(WgradFp8Args w) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_sa[C::NST * C::NT];
  __shared__ __attribute__((aligned(16))) float lds_sb[C::NST * C::NT];
  __shared__ int sq[kMaxGroups + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  const int ng = w.E + (w.shared ? 1 : 0);
  for (int i = tid; i <= ng; i += C::NT) sq[i] = w.qtiles[i];
  __syncthreads();
  const int tm = (w.M + C::BM - 1) / C::BM, tn = (w.N + C::BN - 1) / C::BN;
  const int tms = (w.Ms + C::BM - 1) / C::BM, tns = (w.Ns + C::BN - 1) / C::BN;
  const int tpg = tm * tn;
  const int total = w.E * tpg + (w.shared ? tms * tns : 0);
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const int64_t routed_blocks = sq[w.E];

  struct Coord {
    int g, mt, nt, M, N, q0, mtg;
  };
  auto coord = [&](int tile) {
    Coord c;
    int ntn, rem;
    if (tile < w.E * tpg) {
      c.g = tile / tpg;
      rem = tile - c.g * tpg;
      c.M = w.M;
      c.N = w.N;
      ntn = tn;
    } else {
      c.g = w.E;
      rem = tile - w.E * tpg;
      c.M = w.Ms;
      c.N = w.Ns;
      ntn = tns;
    }
    // n fastest: the tiles one XCD runs together write adjacent pieces of the
    // same output rows
    c.mt = rem / ntn;
    c.nt = rem - c.mt * ntn;
    c.q0 = __builtin_amdgcn_readfirstlane(sq[c.g]);
    c.mtg = __builtin_amdgcn_readfirstlane(sq[c.g + 1]) - c.q0;
    return c;
  };
  auto next_ops = [&](int tile, int, StreamOps8<C>& op) {
    const Coord c = coord(tile);
    const bool sh = c.g == w.E;
    const uint32_t npad = static_cast<uint32_t>(c.mtg) * 128u;
    // group bases: routed group g at rows x 128 sq[g]; the shared group after
    // all routed blocks, with its own row count
    const int64_t abase = sh ? static_cast<int64_t>(w.M) * 128 * routed_blocks
                             : static_cast<int64_t>(w.M) * 128 * c.q0;
    const int64_t bbase = sh ? static_cast<int64_t>(w.N) * 128 * routed_blocks
                             : static_cast<int64_t>(w.N) * 128 * c.q0;
    const int64_t asb = sh ? static_cast<int64_t>(w.M) * routed_blocks
                           : static_cast<int64_t>(w.M) * c.q0;
    const int64_t bsb = sh ? static_cast<int64_t>(w.N) * routed_blocks
                           : static_cast<int64_t>(w.N) * c.q0;
    op.ra = rsrc4(w.a + abase, static_cast<uint32_t>(c.M) * npad);
    op.rb = rsrc4(w.b + bbase, static_cast<uint32_t>(c.N) * npad);
    op.rsa = rsrc4(w.as + asb, static_cast<uint32_t>(c.M) * c.mtg * 4u);
    op.rsb = rsrc4(w.bs + bsb, static_cast<uint32_t>(c.N) * c.mtg * 4u);
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int row = c.mt * C::BM + r0 + p * C::RPP;
      op.ao[p] = row < c.M ? static_cast<uint32_t>(row) * npad : kInvalidRow;
    }
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = c.nt * C::BN + r0 + p * C::RPP;
      op.bo[p] = row < c.N ? static_cast<uint32_t>(row) * npad : kInvalidRow;
    }
    const int ra_row = c.mt * C::BM + tid, rb_row = c.nt * C::BN + tid;
    op.sa_off = (tid < C::BM && ra_row < c.M) ? static_cast<uint32_t>(ra_row) * 4u : kInvalidRow;
    op.sb_off = (tid < C::BN && rb_row < c.N) ? static_cast<uint32_t>(rb_row) * 4u : kInvalidRow;
    op.sa_step = static_cast<uint32_t>(c.M) * 4u;  // k-block-major scales
    op.sb_step = static_cast<uint32_t>(c.N) * 4u;
    op.sb_lo = op.sb_hi = 0;
    swizzle_rows8<C>(op.ao);
    swizzle_rows8<C>(op.bo);
    op.nk = c.mtg > 0 ? c.mtg : 1;
  };
  auto nk_of = [&](int tile) {
    const Coord c = coord(tile);
    return c.mtg > 0 ? c.mtg : 1;
  };
  // acc in the A-first layout: lane l owns output column l % 32 of each 32 x 32
  // product and rows 8 g + 4 (l / 32) + q, so one register across the wave
  // stores two 128-byte row pieces. Buffer stores with out-of-range offsets
  // for the masked entries: every call issues exactly MI * NJ * 16 stores (no
  // branch skips one), which lets them drain during the next tile's first k
  // block. The gradients (as large as the weights, in fp32) are written with
  // the non-temporal policy, so that they do not push the operands out of L2.
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const Coord c = coord(tile);
    float* out = c.g < w.E ? w.out + static_cast<int64_t>(c.g) * w.M * w.N : w.out_s;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        out, 0, static_cast<int>(static_cast<uint32_t>(c.M) * c.N * 4u), 0x00020000);
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) {
      const int n = c.nt * C::BN + wn * C::WN + nj * 32 + (lane & 31);
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
        const int m0 = c.mt * C::BM + wm * C::WM + mi * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 8 * (r >> 2) + (r & 3);
          const uint32_t off = (m < c.M && n < c.N)
                                   ? (static_cast<uint32_t>(m) * c.N + n) * 4u
                                   : kInvalidRow;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[mi][nj][r]), ro, off, 0,
                                                kNonTemporal);
        }
      }
    }
  };
  constexpr int kStores = C::MI * C::NJ * 16;
  constexpr int kIn = C::template NL<true> * (C::NST - 2);
  constexpr int kPost = kIn + kStores < 63 ? kIn + kStores : 63;
  static_assert(kPost <= kStores + kIn, "the waits after an epilogue stay exact");
  gemm8_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, FB, FA,
               true, false, kPost>(lds, lds_sa, lds_sb, first, nb, total, next_ops, nk_of,
                                   epilogue);
}

// ---- 128x1 quantization along the tokens, written transposed ----------------
//
// One workgroup per 128-row block of a group and 64 channels: the block's
// rows (routed: rows offsets[g] .. of src, or of x through perm; shared:
// rows of src_s) go through LDS; each channel's max-abs over the 128 rows
// gives its scale, and its 128 codes leave as one contiguous run of the
// transposed [channels, tokens] layout. Rows past the group's end are zeros.
template <int FMT>
__global__ __launch_bounds__(256) void quant_cols_kernel(QuantColsArgs q) {
  __shared__ float tile[128][65];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int total = q.qtiles[q.E + (q.shared ? 1 : 0)];
  if (t >= total) return;
  // group of block t: the last g with qtiles[g] <= t
  int lo = 0, hi = q.E + (q.shared ? 1 : 0);
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (q.qtiles[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const bool sh = q.shared && g == q.E;
  const int C = sh ? q.Cs : q.C;
  const int c0 = blockIdx.y * 64;
  if (c0 >= C) return;
  const int q0 = q.qtiles[g], mtg = q.qtiles[g + 1] - q0;
  const int blk = t - q0;
  const int64_t rows = sh ? q.T : q.offsets[g + 1] - q.offsets[g];
  // load 128 rows x 64 channels (bf16): 8 threads per row, 16 bytes each
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = (tid >> 3) + 32 * p;
    const int j = tid & 7;
    const int64_t r = static_cast<int64_t>(blk) * 128 + i;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r < rows) {
      const uint16_t* src;
      if (sh) {
        src = q.src_s + r * q.ld_s;
      } else {
        const int64_t pos = q.offsets[g] + r;
        src = q.perm ? q.src + static_cast<int64_t>(q.perm[pos]) * q.ld : q.src + pos * q.ld;
      }
      const uint4 u = *reinterpret_cast<const uint4*>(src + c0 + 8 * j);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(wv[k] << 16);
        v[2 * k + 1] = __uint_as_float(wv[k] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[i][8 * j + k] = v[k];
  }
  __syncthreads();
  // channel ch = tid / 4, rows 32 s .. 32 s + 31 with s = tid % 4
  const int ch = tid >> 2, s = tid & 3;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    v[k] = tile[32 * s + k][ch];
    amax = fmaxf(amax, fabsf(v[k]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const float inv = amax == 0.0f ? 0.0f : Fp8Fmt<FMT>::kMax / amax;
  uint32_t w4[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    w4[k] = amax == 0.0f ? 0u
                         : Fp8Fmt<FMT>::pack4(v[4 * k] * inv, v[4 * k + 1] * inv,
                                              v[4 * k + 2] * inv, v[4 * k + 3] * inv);
  const int64_t routed_blocks = q.qtiles[q.E];
  const int64_t cb = sh ? static_cast<int64_t>(q.C) * 128 * routed_blocks
                        : static_cast<int64_t>(q.C) * 128 * q0;
  const int64_t sbase = sh ? static_cast<int64_t>(q.C) * routed_blocks
                           : static_cast<int64_t>(q.C) * q0;
  const int64_t npad = static_cast<int64_t>(mtg) * 128;
  uint8_t* dst = q.q + cb + static_cast<int64_t>(c0 + ch) * npad + blk * 128 + 32 * s;
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(w4[4], w4[5], w4[6], w4[7]);
  // scales k-block major inside the group ([blocks, channels]): a tile's
  // channel scales of one token block are one contiguous run
  if (s == 0) q.scale[sbase + static_cast<int64_t>(blk) * C + c0 + ch] =
      amax == 0.0f ? 1.0f : amax / Fp8Fmt<FMT>::kMax;
}

// ---- transposed copies of FP8 weights ---------------------------------------
//
// codes [n, R, C] -> [n, C, R] through 64 x 64 byte tiles in LDS.
__global__ __launch_bounds__(256) void transpose_codes_kernel(const uint8_t* __restrict__ src,
                                                              int R, int C,
                                                              uint8_t* __restrict__ dst) {
  __shared__ uint8_t tile[64][64 + 4];
  const int tid = threadIdx.x;
  const int tr = R / 64, tc = C / 64;
  const int64_t b = blockIdx.x;
  const int64_t mat = b / (static_cast<int64_t>(tr) * tc);
  const int bi = static_cast<int>((b / tc) % tr), bj = static_cast<int>(b % tc);
  const uint8_t* s = src + mat * R * static_cast<int64_t>(C);
  uint8_t* d = dst + mat * R * static_cast<int64_t>(C);
  {
    const int i = tid >> 2, j = (tid & 3) * 16;
    const uint4 u = *reinterpret_cast<const uint4*>(s + static_cast<int64_t>(bi * 64 + i) * C +
                                                    bj * 64 + j);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[i][j + k] = static_cast<uint8_t>(w[k >> 2] >> (8 * (k & 3)));
  }
  __syncthreads();
  {
    const int i = tid >> 2, j = (tid & 3) * 16;  // output row i (source column), 16 rows of it
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k >> 2] |= static_cast<uint32_t>(tile[j + k][i]) << (8 * (k & 3));
    *reinterpret_cast<uint4*>(d + static_cast<int64_t>(bj * 64 + i) * R + bi * 64 + j) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// scales [n, rb, cb] -> [n, cb, rb]
__global__ __launch_bounds__(256) void transpose_scales_kernel(const float* __restrict__ src,
                                                               int64_t n, int rb, int cb,
                                                               float* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n * rb * cb) return;
  const int64_t mat = i / (static_cast<int64_t>(rb) * cb);
  const int r = static_cast<int>((i / cb) % rb), c = static_cast<int>(i % cb);
  dst[mat * rb * cb + static_cast<int64_t>(c) * rb + r] = src[i];
}

}  // namespace

hipError_t launch_dgrad2_fp8(const BwdFp8Args& a, hipStream_t s) {
  using C = T8Bwd;
  static int occ = 0;
  if (!occ) occ = occupancy_fp8b(dgrad2_fp8_kernel<C>, C::NT);
  const int g = ((device_cu_count() * occ + 7) / 8) * 8;
  hipLaunchKernelGGL(dgrad2_fp8_kernel<C>, dim3(g), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dgrad1_fp8(const BwdFp8Args& a, hipStream_t s) {
  using C = T8Bwd;
  static int occ = 0;
  if (!occ) occ = occupancy_fp8b(dgrad1_fp8_kernel<C>, C::NT);
  const int g = ((device_cu_count() * occ + 7) / 8) * 8;
  hipLaunchKernelGGL(dgrad1_fp8_kernel<C>, dim3(g), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_wgrad_fp8(const WgradFp8Args& w, int fa, int fb, hipStream_t s) {
  using C = T8Bwd;
  if (fa == kE5M2 && fb == kE4M3) {
    static int occ = 0;
    if (!occ) occ = occupancy_fp8b(wgrad_fp8_kernel<C, kE5M2, kE4M3>, C::NT);
    const int g = ((device_cu_count() * occ + 7) / 8) * 8;
    hipLaunchKernelGGL((wgrad_fp8_kernel<C, kE5M2, kE4M3>), dim3(g), dim3(C::NT), 0, s, w);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quant_cols(const QuantColsArgs& q, int64_t max_blocks, int fmt, hipStream_t s) {
  if (max_blocks == 0) return hipSuccess;
  const int cmax = q.C > q.Cs ? q.C : q.Cs;
  const dim3 grid(static_cast<unsigned>(max_blocks), static_cast<unsigned>((cmax + 63) / 64));
  if (fmt == kE5M2)
    hipLaunchKernelGGL(quant_cols_kernel<kE5M2>, grid, dim3(256), 0, s, q);
  else
    hipLaunchKernelGGL(quant_cols_kernel<kE4M3>, grid, dim3(256), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_transpose_fp8(const uint8_t* q, const float* scale, int64_t n_mats, int rows,
                                int cols, uint8_t* qt, float* scale_t, hipStream_t s) {
  const int64_t tiles = n_mats * (rows / 64) * static_cast<int64_t>(cols / 64);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_codes_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s, q,
                     rows, cols, qt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t ns = n_mats * (rows / 128) * static_cast<int64_t>(cols / 128);
  hipLaunchKernelGGL(transpose_scales_kernel, dim3(static_cast<unsigned>((ns + 255) / 256)),
                     dim3(256), 0, s, scale, n_mats, rows / 128, cols / 128, scale_t);
  return hipGetLastError();
}

}  // namespace dsmoe
