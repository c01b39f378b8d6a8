// Backward of the DeepSeekMoE feed-forward layer on gfx950 for bf16
// activations and weights: fp32 accumulation everywhere, fp32 weight
// gradients (the pages keep weight gradients in high precision: mhpq.cn
// "DeepSeek-V3 高效训练关键技术全景解析" §4.1), bf16 intermediates like the
// forward's.
//
// For a fixed selection the layer is y_t = FFN_s(x_t) + sum_k g_tk FFN_e(x_t)
// with g = s / S over the selected sigmoid scores (kaiyunto.com DeepSeek-V3
// walkthrough, DeepSeekMoE paragraph; mhpq.cn §1.1); the selection bias gets
// no gradient (it follows the load rule, mhpq.cn §1.2). The steps:
//   gate:    dg_tk = <dy_t, y_perm[r]>, dYp[r] = g_tk dy_t (r = inv[t,k]),
//            du_tk = (dg_tk - sum_j g_tj dg_tj) / S_t * s_tk (1 - s_tk);
//   dgrad2:  dH = dYp W2_e (shared: dy Ws2), then the SwiGLU backward
//            da = dH b silu'(a), db = dH silu(a) from the saved a, b;
//   dgrad1:  dA = [da | db] [W1_e; W3_e];
//            both contract over the weights' output rows and read the
//            weights in their forward layout as k-major operands (LDS
//            transpose reads, see gemm_bf16_core.h);
//   combine: dx_t = dA_s[t] + sum_k dA[inv[t,k]] + sum_k du_tk Wr[e_tk];
//   router:  dWr[e] = sum over e's rows of du x;
//   wgrad:   dW13_e = [da | db]_e^T A_e, dW2_e = dYp_e^T H_e, as GEMMs whose
//            contraction runs over the expert's tokens: both operands are
//            read k-major from their row layouts (A_e from a gathered copy
//            of x), each bounded to the expert's rows.
#include "device_common.h"
#include "internal.h"
#include "tile_schedule.h"
#include "gemm_bf16_core.h"
#include "sigmoid_ieee.h"

namespace dsmoe {

namespace {

// ---- gate and router gradients -------------------------------------------

constexpr int kRowT = 256;

__device__ __forceinline__ float block_sum4(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

// One workgroup per token t: dg_tk = <dy_t, y_perm[inv[t,k]]> (fp32, fixed
// order), dYp[inv[t,k]] = bf16(g_tk dy_t), then the router gradient of the
// selected logits du_tk (also scattered to permuted order as du_perm).
__global__ __launch_bounds__(kRowT) void bwd_gate_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ yperm,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ inv,
    const float* __restrict__ gate, const float* __restrict__ logits, int K, int E, int d,
    uint16_t* __restrict__ dyp, float* __restrict__ du, float* __restrict__ du_perm) {
  __shared__ float red[4];
  __shared__ float dg[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = d / 8;
  const uint16_t* dyr = dy + t * d;
  for (int k = 0; k < K; ++k) {
    const int64_t r = inv[t * K + k];
    const float g = gate[t * K + k];
    const uint16_t* yr = yperm + r * d;
    uint16_t* outr = dyp + r * d;
    float acc = 0.0f;
    for (int ch = tid; ch < nch; ch += kRowT) {
      const uint4 a = *reinterpret_cast<const uint4*>(dyr + ch * 8);
      const uint4 b = *reinterpret_cast<const uint4*>(yr + ch * 8);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
      uint32_t ow[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = __uint_as_float(aw[j] << 16), a1 = __uint_as_float(aw[j] & 0xFFFF0000u);
        const float b0 = __uint_as_float(bw[j] << 16), b1 = __uint_as_float(bw[j] & 0xFFFF0000u);
        acc += a0 * b0;
        acc += a1 * b1;
        ow[j] = pack_bf16x2(g * a0, g * a1);
      }
      *reinterpret_cast<uint4*>(outr + ch * 8) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
    const float s = block_sum4(acc, red);
    if (tid == 0) dg[k] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float S = 0.0f, mean = 0.0f;
    for (int k = 0; k < K; ++k) {
      S += sigmoid_ieee(logits[t * E + idx[t * K + k]]);
      mean += gate[t * K + k] * dg[k];
    }
    for (int k = 0; k < K; ++k) {
      const float s = sigmoid_ieee(logits[t * E + idx[t * K + k]]);
      const float v = S > 0.0f ? (dg[k] - mean) / S * (s * (1.0f - s)) : 0.0f;
      du[t * K + k] = v;
      du_perm[inv[t * K + k]] = v;
    }
  }
}

// dx_t = dA_s[t] + sum_k dA[inv[t,k]] + sum_k du_tk Wr[idx[t,k]], fp32 in that
// order, bf16 out. One workgroup per token.
constexpr int kRowsInFlight = 8;

__global__ __launch_bounds__(kRowT) void bwd_combine_kernel(
    const uint16_t* __restrict__ dap, const uint16_t* __restrict__ das,
    const int32_t* __restrict__ inv, const int32_t* __restrict__ idx,
    const float* __restrict__ du, const float* __restrict__ wr, int K, int d,
    uint16_t* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  const int nch = d / 8;
  for (int ch = threadIdx.x; ch < nch; ch += kRowT) {
    float acc[8];
    if (das) {
      const uint4 v = *reinterpret_cast<const uint4*>(das + t * d + ch * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = __uint_as_float(w[j] << 16);
        acc[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    }
    // the rows' loads go out eight at a time, then add in k order
    for (int k0 = 0; k0 < K; k0 += kRowsInFlight) {
      uint4 rv[kRowsInFlight];
#pragma unroll
      for (int k = 0; k < kRowsInFlight; ++k)
        if (k0 + k < K)
          rv[k] = *reinterpret_cast<const uint4*>(
              dap + static_cast<int64_t>(inv[t * K + k0 + k]) * d + ch * 8);
#pragma unroll
      for (int k = 0; k < kRowsInFlight; ++k) {
        if (k0 + k >= K) break;
        const uint32_t w[4] = {rv[k].x, rv[k].y, rv[k].z, rv[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += __uint_as_float(w[j] << 16);
          acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
        }
      }
    }
    for (int k = 0; k < K; ++k) {
      const float u = du[t * K + k];
      const float* wrow = wr + static_cast<int64_t>(idx[t * K + k]) * d + ch * 8;
      const float4 lo = *reinterpret_cast<const float4*>(wrow);
      const float4 hi = *reinterpret_cast<const float4*>(wrow + 4);
      acc[0] += u * lo.x; acc[1] += u * lo.y; acc[2] += u * lo.z; acc[3] += u * lo.w;
      acc[4] += u * hi.x; acc[5] += u * hi.y; acc[6] += u * hi.z; acc[7] += u * hi.w;
    }
    *reinterpret_cast<uint4*>(dx + t * d + ch * 8) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

// dWr[e, j] = sum over the rows r of e's segment, ascending, of
// du_perm[r] * x[perm[r], j], fp32. Grid (ceil(d / 2048), E); 8 columns per
// thread.
__global__ __launch_bounds__(kRowT) void router_wgrad_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const float* __restrict__ du_perm, int d,
    float* __restrict__ dwr) {
  const int e = blockIdx.y;
  const int ch = blockIdx.x * kRowT + threadIdx.x;
  if (ch * 8 >= d) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add_row = [&](float u, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += u * __uint_as_float(w[j] << 16);
      acc[2 * j + 1] += u * __uint_as_float(w[j] & 0xFFFF0000u);
    }
  };
  const uint16_t* xc = x + ch * 8;
  const int r1 = offsets[e + 1];
  int r = offsets[e];
  // sixteen rows in flight per iteration (the hottest expert's segment bounds
  // the kernel); they are added in row order
  for (; r + 16 <= r1; r += 16) {
    uint4 v[16];
    float u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] = *reinterpret_cast<const uint4*>(xc + static_cast<int64_t>(perm[r + i]) * d);
      u[i] = du_perm[r + i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) add_row(u[i], v[i]);
  }
  for (; r < r1; ++r)
    add_row(du_perm[r], *reinterpret_cast<const uint4*>(xc + static_cast<int64_t>(perm[r]) * d));
  float* out = dwr + static_cast<int64_t>(e) * d + ch * 8;
  *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// ---- grouped GEMMs -----------------------------------------------------------

// dH = dYp W2_e per routed group (rows of the group's segment) and dy Ws2 for
// the shared group, W2 read in its forward layout [d, I] as a k-major
// operand, then the SwiGLU backward from the saved pre-activations:
// dG = [da | db].
template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void dgrad2_bf16_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ GroupTables gt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles, a.offsets, a.E);
  const int total = gt.total;
  // one tile per workgroup (long k loops: d / 64 steps), XCD-contiguous
  const int first = xcd_single_tile(blockIdx.x, total);
  if (first < 0) return;
  const int nb = total;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const int nk = a.d / BK;
  const int64_t ldg = 2 * static_cast<int64_t>(a.ldh);

  auto next_ops = [&](int tile, int, StreamOps<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int rows_left = c.rows - c.m * C::BM;
    const int64_t rbase = (c.shared ? 0 : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    // the tile's gradient rows through a resource based at its first row
    // (64-bit base, 32-bit offsets inside the tile)
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left ? static_cast<uint32_t>(lr) * row_bytes : kInvalidRow;
    }
    op.ra = rsrc4(static_cast<const uint16_t*>(c.shared ? a.dy : a.dyp) + rbase * a.d,
                  static_cast<uint32_t>(rows_left < C::BM ? rows_left : C::BM) * row_bytes);
    swizzle_rows<C>(op.ao);
    const uint16_t* W = c.shared ? static_cast<const uint16_t*>(a.ws2)
                                 : static_cast<const uint16_t*>(a.w2) +
                                       static_cast<int64_t>(c.g) * a.d * a.I;
    const uint32_t ld_bytes = static_cast<uint32_t>(Ig) * 2u;
    op.rb = rsrc4(W, static_cast<uint32_t>(a.d) * ld_bytes);
    // columns past Ig (last column tile) read neighbouring data or zeros;
    // they only reach output columns that are not stored
    kmajor_offsets<C::BN, C::B_LOADS, C::NT>(op.bo, c.n * C::BN, ld_bytes);
    op.kstep_b = BK * ld_bytes;
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
      const uint16_t* gp = static_cast<const uint16_t*>(a.gu) + (hrow0 + row) * ldg;
      uint16_t* dp = static_cast<uint16_t*>(a.dg) + (hrow0 + row) * ldg;
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = c.n * C::BN + wn * C::WN + nj * 32 + 8 * g + 4 * (lane >> 5);
          if (col >= Ig) continue;
          const uint2 av = *reinterpret_cast<const uint2*>(gp + col);
          const uint2 bv = *reinterpret_cast<const uint2*>(gp + Ig + col);
          const uint32_t aw[2] = {av.x, av.y}, bw[2] = {bv.x, bv.y};
          float da[4], db[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t ab = (j & 1) ? (aw[j >> 1] & 0xFFFF0000u) : (aw[j >> 1] << 16);
            const uint32_t bb = (j & 1) ? (bw[j >> 1] & 0xFFFF0000u) : (bw[j >> 1] << 16);
            const float x = __uint_as_float(ab), u = __uint_as_float(bb);
            const float dh = acc[mi][nj][4 * g + j];
            const float sg = 1.0f / (1.0f + __expf(-x));
            da[j] = dh * u * (sg * (1.0f + x * (1.0f - sg)));
            db[j] = dh * (x * sg);
          }
          *reinterpret_cast<uint2*>(dp + col) =
              make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
          *reinterpret_cast<uint2*>(dp + Ig + col) =
              make_uint2(pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3]));
        }
    }
  };
  gemm_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, true, -1, true>(
      lds, first, nb, total, next_ops, nk_of, epilogue);
}

// dA = [da | db] [W1_e; W3_e] per routed group and the same with the shared
// weights for the shared rows: the contraction runs over the 2 Ig rows of
// W13 [2Ig, d], read in its forward layout as a k-major operand. bf16 out.
template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void dgrad1_bf16_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ GroupTables gt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  load_group_tables(gt, a.tiles, a.offsets, a.E);
  const int total = gt.total;
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;
  const uint32_t grow_bytes = static_cast<uint32_t>(a.ldh) * 4u;  // rows of [da | db]
  const uint32_t ld_bytes = static_cast<uint32_t>(a.d) * 2u;
  const int shared_first = a.E > 0 ? gt.gnext[a.E - 1] : 0;

  auto next_ops = [&](int tile, int, StreamOps<C>& op) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int Ig = c.shared ? a.Is : a.I;
    const int64_t hrow0 = (c.shared ? a.TK : c.rbase) + static_cast<int64_t>(c.m) * C::BM;
    const int rows_left = c.rows - c.m * C::BM;
    // the tile's [da | db] rows through a resource based at its first row
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      op.ao[p] = lr < rows_left ? static_cast<uint32_t>(lr) * grow_bytes : kInvalidRow;
    }
    op.ra = rsrc4(static_cast<const uint16_t*>(a.dg) + hrow0 * 2 * a.ldh,
                  static_cast<uint32_t>(rows_left < C::BM ? rows_left : C::BM) * grow_bytes);
    swizzle_rows<C>(op.ao);
    const uint16_t* W = c.shared ? static_cast<const uint16_t*>(a.ws13)
                                 : static_cast<const uint16_t*>(a.w13) +
                                       static_cast<int64_t>(c.g) * 2 * a.I * a.d;
    op.rb = rsrc4(W, static_cast<uint32_t>(2 * Ig) * ld_bytes);
    kmajor_offsets<C::BN, C::B_LOADS, C::NT>(op.bo, c.n * C::BN, ld_bytes);
    op.kstep_b = BK * ld_bytes;
    op.nk = 2 * Ig / BK;
  };
  auto nk_of = [&](int tile) { return 2 * (tile >= shared_first ? a.Is : a.I) / BK; };
  auto epilogue = [&](int tile, f32x16_t (&acc)[C::MI][C::NJ]) {
    const TileCoord c = tile_coord_lds(gt, a.E, a.T, tile, C::BM);
    const int rows_left = c.rows - c.m * C::BM;
    uint16_t* out = c.shared ? static_cast<uint16_t*>(a.das) +
                                   static_cast<int64_t>(c.m) * C::BM * a.d
                             : static_cast<uint16_t*>(a.dap) +
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
          *reinterpret_cast<uint2*>(yp + col) = pack_bf16x4(v[4 * g], v[4 * g + 1],
                                                            v[4 * g + 2], v[4 * g + 3]);
        }
    }
  };
  gemm_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, true, -1, true>(
      lds, first, nb, total, next_ops, nk_of, epilogue);
}

// Weight gradients out_g = A_g^T B_g (fp32) per group g, contracting over
// the group's rows (tokens): A_g = rows offsets[g] .. offsets[g+1] - 1 of a
// (the shared group: rows 0 .. T - 1 of a_s), columns m < M_g; B_g likewise
// from b / b_s, columns n < N_g. Both operands are k-major (a k-step is 64
// consecutive rows) and read by transpose reads. Each group's operands are
// buffer resources that start at the group's first row and end at its last,
// so the rows of the last k-step past the segment read as zeros in hardware
// (an empty group reads one k-step of zeros and stores zeros).
// Tiles: ceil(M/BM) x ceil(N/BN) per group, routed groups first, the shared
// group last; inside a group, rows of kSuperM m-tiles, m fastest: the 32
// consecutive tiles one XCD runs at a time read 8 A panels and 4 B panels,
// where an n-fastest order reads one A panel against every B panel of the
// expert, more than the L2 keeps, once per m-tile.
constexpr int kSuperM = 8;

template <class C>
__global__ __launch_bounds__(C::NT, C::MINW) void wgrad_bf16_kernel(WgradArgs w) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ int soff[kMaxGroups + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  for (int i = tid; i <= w.E; i += C::NT) soff[i] = w.offsets[i];
  __syncthreads();
  const int tn = (w.N + C::BN - 1) / C::BN, tm = (w.M + C::BM - 1) / C::BM, tpr = tm * tn;
  const int tns = (w.Ns + C::BN - 1) / C::BN, tms = (w.Ms + C::BM - 1) / C::BM;
  const int total = w.E * tpr + (w.shared ? tms * tns : 0);
  const int nb = gridDim.x;
  const int first = xcd_logical_block(blockIdx.x, nb);
  if (first >= total) return;

  struct Coord {
    int g, mt, nt, M, N, rows, row0;
  };
  auto coord = [&](int tile) {
    Coord c;
    int rem, ntm, ntn;
    if (tile < w.E * tpr) {
      c.g = tile / tpr;
      rem = tile - c.g * tpr;
      c.M = w.M;
      c.N = w.N;
      // wave-uniform: the operands' buffer descriptors live in scalar registers
      c.row0 = __builtin_amdgcn_readfirstlane(soff[c.g]);
      c.rows = __builtin_amdgcn_readfirstlane(soff[c.g + 1]) - c.row0;
      ntm = tm;
      ntn = tn;
    } else {
      rem = tile - w.E * tpr;
      c.g = w.E;
      c.M = w.Ms;
      c.N = w.Ns;
      c.row0 = 0;
      c.rows = static_cast<int>(w.T);
      ntm = tms;
      ntn = tns;
    }
    const int per_row = kSuperM * ntn;
    const int gr = rem / per_row;
    const int r2 = rem - gr * per_row;
    const int sm = min(kSuperM, ntm - gr * kSuperM);
    c.nt = r2 / sm;
    c.mt = gr * kSuperM + (r2 - c.nt * sm);
    return c;
  };
  auto k_steps = [](int rows) { return rows > BK ? (rows + BK - 1) / BK : 1; };
  auto next_ops = [&](int tile, int, StreamOps<C>& op) {
    const Coord c = coord(tile);
    const bool sh = c.g == w.E;
    const uint16_t* A = static_cast<const uint16_t*>(sh ? w.a_s : w.a);
    const uint16_t* B = static_cast<const uint16_t*>(sh ? w.b_s : w.b);
    const int64_t lda = sh ? w.lda_s : w.lda, ldb = sh ? w.ldb_s : w.ldb;
    const uint32_t la = static_cast<uint32_t>(lda) * 2u, lb = static_cast<uint32_t>(ldb) * 2u;
    op.ra = rsrc4(A + c.row0 * lda, static_cast<uint32_t>(c.rows) * la);
    op.rb = rsrc4(B + c.row0 * ldb, static_cast<uint32_t>(c.rows) * lb);
    kmajor_offsets<C::BM, C::A_LOADS, C::NT>(op.ao, c.mt * C::BM, la);
    kmajor_offsets<C::BN, C::B_LOADS, C::NT>(op.bo, c.nt * C::BN, lb);
    op.kstep_a = BK * la;
    op.kstep_b = BK * lb;
    op.nk = k_steps(c.rows);
  };
  auto nk_of = [&](int tile) { return k_steps(coord(tile).rows); };
  // acc in the unswapped layout: lane l owns column l % 32 of each 32 x 32
  // product, so one register across the wave stores two 128-byte row pieces.
  // Buffer stores with out-of-range offsets for the masked entries: every
  // call issues exactly MI * NJ * 16 stores (no branch can skip one), which
  // with three stages lets them drain during the next tile's first step.
  // Non-temporal: the call does not read these outputs again (backward 24.2
  // -> 23.7 ms at V3 shape).
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
        const int m0 = c.mt * C::BM + wm * C::WM + mi * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + acc_row(lane, r);
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
  constexpr int kPost =
      C::NST < 3 ? -1 : kInflight<C> + kStores < 63 ? kInflight<C> + kStores : 63;
  gemm_stream<C, false, decltype(next_ops)&, decltype(nk_of)&, decltype(epilogue)&, false, kPost,
              true, true>(lds, first, nb, total, next_ops, nk_of, epilogue);
}

template <class K>
int occupancy_of(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

}  // namespace

hipError_t launch_bwd_gate(const void* dy, const void* yperm, const int32_t* idx,
                           const int32_t* inv, const float* gate, const float* logits, int64_t T,
                           int K, int E, int d, void* dyp, float* du, float* du_perm,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_gate_kernel, dim3(static_cast<unsigned>(T)), dim3(kRowT), 0, s,
                     static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(yperm), idx,
                     inv, gate, logits, K, E, d, static_cast<uint16_t*>(dyp), du, du_perm);
  return hipGetLastError();
}

hipError_t launch_bwd_combine(const void* dap, const void* das, const int32_t* inv,
                              const int32_t* idx, const float* du, const float* wr, int64_t T,
                              int K, int d, void* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3(static_cast<unsigned>(T)), dim3(kRowT), 0, s,
                     static_cast<const uint16_t*>(dap), static_cast<const uint16_t*>(das), inv,
                     idx, du, wr, K, d, static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const void* x, const int32_t* perm, const int32_t* offsets,
                               const float* du_perm, int E, int d, float* dwr, hipStream_t s) {
  dim3 grid((d / 8 + kRowT - 1) / kRowT, E);
  hipLaunchKernelGGL(router_wgrad_kernel, grid, dim3(kRowT), 0, s,
                     static_cast<const uint16_t*>(x), perm, offsets, du_perm, d, dwr);
  return hipGetLastError();
}

// more than the tiles of the plan: routed rows in 128-row tiles (at most
// ceil(TK / 128) + E m-tiles over all groups) and the shared rows
int64_t dgrad_tile_bound(const BwdArgs& a, int n_routed, int n_shared) {
  const int64_t m = (a.TK + 127) / 128 + a.E;
  const int64_t b = m * n_routed + (a.Is > 0 ? (a.T + 127) / 128 * n_shared : 0);
  return (b + 7) / 8 * 8;
}

hipError_t launch_dgrad2_bf16(const BwdArgs& a, hipStream_t s) {
  using C = TilePrefill;
  const int g = static_cast<int>(dgrad_tile_bound(a, (a.I + C::BN - 1) / C::BN,
                                                  (a.Is + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(dgrad2_bf16_kernel<C>, dim3(g), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dgrad1_bf16(const BwdArgs& a, hipStream_t s) {
  using C = TilePrefill;
  static int occ = 0;
  if (!occ) occ = occupancy_of(dgrad1_bf16_kernel<C>, C::NT);
  const int g = ((device_cu_count() * occ + 7) / 8) * 8;
  hipLaunchKernelGGL(dgrad1_bf16_kernel<C>, dim3(g), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

// Weight-gradient tiles of 256 x 256 (8 waves of 64 x 128) with a two-stage
// ring (128 KB; three stages would need 192 KB): each CU moves its loads and
// its fp32 stores through one memory pipeline, and this tile loads a third
// fewer bytes per output than 128 x 256 (backward 23.5-24.0 -> 22.8-23.2 ms
// at V3 shape, same results bit for bit).
using TileWgrad = Tile<256, 256, 64, 128, 2>;

hipError_t launch_wgrad_bf16(const WgradArgs& w, hipStream_t s) {
  using C = TileWgrad;
  static int occ = 0;
  if (!occ) occ = occupancy_of(wgrad_bf16_kernel<C>, C::NT);
  const int g = ((device_cu_count() * occ + 7) / 8) * 8;
  hipLaunchKernelGGL(wgrad_bf16_kernel<C>, dim3(g), dim3(C::NT), 0, s, w);
  return hipGetLastError();
}

}  // namespace dsmoe
