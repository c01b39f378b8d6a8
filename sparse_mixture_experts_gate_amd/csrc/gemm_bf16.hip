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

namespace dsmoe {

namespace {

constexpr int BK = 64;  // k elements per stage: 128 bytes per row

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int RPP = NT / 8;  // rows covered by one pass of 16-byte loads
  static constexpr int A_LOADS = BM / RPP;
  static constexpr int B_LOADS = BN / RPP;
  static constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per stage
  static constexpr int LDS_ELEMS = 2 * STAGE;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must cover the load passes");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA sub-tiles");
};

using TilePrefill = Tile<128, 128, 64, 64>;  // 4 waves, 64 KB LDS
using TileDecode = Tile<32, 128, 32, 64>;    // 2 waves, 40 KB LDS

// LDS element offset of 16-byte chunk `ch` (0..7) of row `r`.
__device__ __forceinline__ int lds_off(int r, int ch) { return r * BK + ((ch ^ (r & 7)) << 3); }

template <class C, bool SWIGLU>
__device__ __forceinline__ int b_local_row(int wn, int nj) {
  if constexpr (SWIGLU) {
    constexpr int half = C::BN / 2, hw = C::WN / 2, njh = C::NJ / 2;
    return nj < njh ? wn * hw + nj * 32 : half + wn * hw + (nj - njh) * 32;
  } else {
    return wn * C::WN + nj * 32;
  }
}

// acc[mi][nj] += A(rows of arow) * B(rows of brow)^T over k in [k_begin, k_end).
// Row pointers are per thread (the rows this thread loads); nullptr rows read
// as zeros. With a_kmod != 0 the A column is k mod a_kmod (router: the same
// activations meet the three weight terms).
template <class C, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(uint16_t* lds, const uint16_t* const (&arow)[C::A_LOADS],
                                          const uint16_t* const (&brow)[C::B_LOADS], int k_begin,
                                          int k_end, int a_kmod,
                                          f32x16_t (&acc)[C::MI][C::NJ]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int ch = tid & 7, r0 = tid >> 3;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

  uint4 ra[C::A_LOADS], rb[C::B_LOADS];
  auto gload = [&](int k0) {
    const int kc = k0 + ch * 8;
    const bool kin = kc < k_end;
    const int ka = a_kmod ? (k0 % a_kmod) + ch * 8 : kc;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p)
      ra[p] = (arow[p] && kin) ? *reinterpret_cast<const uint4*>(arow[p] + ka)
                               : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p)
      rb[p] = (brow[p] && kin) ? *reinterpret_cast<const uint4*>(brow[p] + kc)
                               : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int st) {
    uint16_t* As = lds + st * C::STAGE;
    uint16_t* Bs = As + C::BM * BK;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p)
      *reinterpret_cast<uint4*>(As + lds_off(r0 + p * C::RPP, ch)) = ra[p];
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p)
      *reinterpret_cast<uint4*>(Bs + lds_off(r0 + p * C::RPP, ch)) = rb[p];
  };

  gload(k_begin);
  sstore(0);
  __syncthreads();
  int st = 0;
  for (int k0 = k_begin; k0 < k_end; k0 += BK) {
    const bool more = k0 + BK < k_end;
    if (more) gload(k0 + BK);
    const uint16_t* As = lds + st * C::STAGE;
    const uint16_t* Bs = As + C::BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chk = kk * 2 + (lane >> 5);
      bf16x8_t af[C::MI], bfr[C::NJ];
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
        const int r = wm * C::WM + mi * 32 + (lane & 31);
        af[mi] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(r, chk));
      }
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) {
        const int r = b_local_row<C, SWIGLU>(wn, nj) + (lane & 31);
        bfr[nj] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(r, chk));
      }
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NJ; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
    }
    if (more) sstore(st ^ 1);
    __syncthreads();
    st ^= 1;
  }
}

// Row (within the tile) of accumulator element r of a 32x32 sub-tile, for
// this lane; the lane's column is lane % 32.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Per tile: group g, row range and column tile n of a grouped GEMM.
struct TileCoord {
  int g, rows, rbase, m, n;
  bool shared;
};

__device__ __forceinline__ TileCoord tile_coord(const FfnArgs& a, const int32_t* tiles,
                                                const int32_t* tmap, int tile, int bm) {
  TileCoord c;
  c.g = tmap[tile];
  c.shared = c.g == a.E;
  c.rbase = c.shared ? 0 : a.offsets[c.g];
  c.rows = c.shared ? static_cast<int>(a.T) : a.offsets[c.g + 1] - c.rbase;
  const int mt = (c.rows + bm - 1) / bm;
  const int local = tile - tiles[c.g];
  c.n = local / mt;
  c.m = local % mt;
  return c;
}

// H = silu(A W1^T) * (A W3^T) per group.
template <class C>
__global__ __launch_bounds__(C::NT) void ffn1_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  constexpr int HALF = C::BN / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  const int total = a.tiles1[a.E + 1];
  const int nb = gridDim.x;
  const uint16_t* X = static_cast<const uint16_t*>(a.perm ? a.x : a.xperm);
  const uint16_t* Xs = static_cast<const uint16_t*>(a.x);
  uint16_t* H = static_cast<uint16_t*>(a.H);
  for (int tile = xcd_logical_block(blockIdx.x, nb); tile < total; tile += nb) {
    const TileCoord tc = tile_coord(a, a.tiles1, a.tmap1, tile, C::BM);
    const int Ig = tc.shared ? a.Is : a.I;
    const uint16_t* arow[C::A_LOADS];
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int r = tc.m * C::BM + r0 + p * C::RPP;
      const uint16_t* ptr = nullptr;
      if (r < tc.rows) {
        if (tc.shared) {
          ptr = Xs + static_cast<int64_t>(r) * a.d;
        } else if (a.perm) {
          const int tok = a.perm[tc.rbase + r];
          ptr = (tok >= 0 && tok < a.T) ? X + static_cast<int64_t>(tok) * a.d : nullptr;
        } else
          ptr = X + static_cast<int64_t>(tc.rbase + r) * a.d;
      }
      arow[p] = ptr;
    }
    const uint16_t* W = tc.shared ? static_cast<const uint16_t*>(a.ws13)
                                  : static_cast<const uint16_t*>(a.w13) +
                                        static_cast<int64_t>(tc.g) * 2 * a.I * a.d;
    const uint16_t* brow[C::B_LOADS];
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      const bool up = lr >= HALF;
      const int col = tc.n * HALF + (up ? lr - HALF : lr);
      brow[p] = col < Ig ? W + static_cast<int64_t>(up ? Ig + col : col) * a.d : nullptr;
    }
    f32x16_t acc[C::MI][C::NJ];
    gemm_tile<C, true>(lds, arow, brow, 0, a.d, 0, acc);

    const int64_t hrow0 = (tc.shared ? a.TK : tc.rbase) + static_cast<int64_t>(tc.m) * C::BM;
    const int rows_left = tc.rows - tc.m * C::BM;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ / 2; ++nj) {
        const int col = tc.n * HALF + wn * (C::WN / 2) + nj * 32 + (lane & 31);
        if (col >= Ig) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * C::WM + mi * 32 + acc_row(lane, r);
          if (lr < rows_left) {
            const float h = silu_f32(acc[mi][nj][r]) * acc[mi][nj + C::NJ / 2][r];
            H[(hrow0 + lr) * a.ldh + col] = f32_to_bf16(h);
          }
        }
      }
  }
}

// y = H W2^T per group: routed rows to y_perm, shared rows to y_shared.
template <class C>
__global__ __launch_bounds__(C::NT) void ffn2_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  const int total = a.tiles2[a.E + 1];
  const int nb = gridDim.x;
  const uint16_t* H = static_cast<const uint16_t*>(a.H);
  for (int tile = xcd_logical_block(blockIdx.x, nb); tile < total; tile += nb) {
    const TileCoord tc = tile_coord(a, a.tiles2, a.tmap2, tile, C::BM);
    const int Ig = tc.shared ? a.Is : a.I;
    const int64_t hrow0 = (tc.shared ? a.TK : tc.rbase) + static_cast<int64_t>(tc.m) * C::BM;
    const int rows_left = tc.rows - tc.m * C::BM;
    const uint16_t* arow[C::A_LOADS];
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lr = r0 + p * C::RPP;
      arow[p] = lr < rows_left ? H + (hrow0 + lr) * a.ldh : nullptr;
    }
    const uint16_t* W = tc.shared ? static_cast<const uint16_t*>(a.ws2)
                                  : static_cast<const uint16_t*>(a.w2) +
                                        static_cast<int64_t>(tc.g) * a.d * a.I;
    const uint16_t* brow[C::B_LOADS];
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int row = tc.n * C::BN + r0 + p * C::RPP;
      brow[p] = row < a.d ? W + static_cast<int64_t>(row) * Ig : nullptr;
    }
    f32x16_t acc[C::MI][C::NJ];
    gemm_tile<C, false>(lds, arow, brow, 0, Ig, 0, acc);

    uint16_t* out = tc.shared ? static_cast<uint16_t*>(a.yshared) +
                                    static_cast<int64_t>(tc.m) * C::BM * a.d
                              : static_cast<uint16_t*>(a.yperm) +
                                    (static_cast<int64_t>(tc.rbase) + tc.m * C::BM) * a.d;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) {
        const int col = tc.n * C::BN + wn * C::WN + nj * 32 + (lane & 31);
        if (col >= a.d) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * C::WM + mi * 32 + acc_row(lane, r);
          if (lr < rows_left) out[static_cast<int64_t>(lr) * a.d + col] = f32_to_bf16(acc[mi][nj][r]);
        }
      }
  }
}

// Router: partial[s][t][e] = sum over k-split s of x[t, k mod d] * wsplit[e, k],
// k in [0, 3d). Grid: (m-tiles * n-tiles, splits).
template <class C>
__global__ __launch_bounds__(C::NT) void router_bf16_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wsplit,
                                                            int64_t T, int d, int E, int kchunk,
                                                            float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r0 = tid >> 3;
  const int ntn = (E + C::BN - 1) / C::BN;
  const int64_t m = blockIdx.x / ntn;
  const int n = blockIdx.x % ntn;
  const int split = blockIdx.y;
  const int k_begin = split * kchunk;
  const int k_end = min(3 * d, k_begin + kchunk);
  const uint16_t* arow[C::A_LOADS];
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) {
    const int64_t t = m * C::BM + r0 + p * C::RPP;
    arow[p] = t < T ? x + t * d : nullptr;
  }
  const uint16_t* brow[C::B_LOADS];
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) {
    const int e = n * C::BN + r0 + p * C::RPP;
    brow[p] = e < E ? wsplit + static_cast<int64_t>(e) * 3 * d : nullptr;
  }
  f32x16_t acc[C::MI][C::NJ];
  gemm_tile<C, false>(lds, arow, brow, k_begin, k_end, d, acc);
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

template <class C>
hipError_t launch_ffn_bf16_cfg(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  static int occ1 = 0, occ2 = 0;
  if (!occ1) occ1 = occupancy_blocks(ffn1_bf16_kernel<C>, C::NT);
  if (!occ2) occ2 = occupancy_blocks(ffn2_bf16_kernel<C>, C::NT);
  const int cus = device_cu_count();
  // persistent grids, multiples of 8 for the XCD remap
  const int g1 = ((cus * occ1 + 7) / 8) * 8;
  const int g2 = ((cus * occ2 + 7) / 8) * 8;
  hipLaunchKernelGGL(ffn1_bf16_kernel<C>, dim3(g1), dim3(C::NT), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(ffn2_bf16_kernel<C>, dim3(g2), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

GemmTiling choose_tiling(int64_t T, int K, int E, int w_dtype) {
  GemmTiling t{};
  const double rows_per_expert = static_cast<double>(T) * K / E;
  if (w_dtype == 2) {  // FP8: 128 intermediate columns per gate/up tile; see gemm_fp8.hip
    if (rows_per_expert < 48.0) {
      t.bm1 = 32; t.bnh1 = 128; t.bm2 = 32; t.bn2 = 128; t.variant = 1;
    } else {
      t.bm1 = 128; t.bnh1 = 128; t.bm2 = 128; t.bn2 = 128; t.variant = 0;
    }
    return t;
  }
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
  if (t.variant == 1) return launch_ffn_bf16_cfg<TileDecode>(a, s, mid);
  return launch_ffn_bf16_cfg<TilePrefill>(a, s, mid);
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
