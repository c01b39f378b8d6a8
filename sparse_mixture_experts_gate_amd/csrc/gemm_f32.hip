// fp32 expert FFNs for fp32 activations and weights: grouped GEMMs on the
// fp32 matrix cores (v_mfma_f32_32x32x2_f32), one wave per 32-row tile of one
// group (mhpq.cn "DeepSeek-V3 高效训练关键技术全景解析" §1.1: the routed experts
// and the shared expert are SwiGLU FFNs). Used for small fp32 layers, where
// single-precision arithmetic matters more than speed: operands come straight
// from global memory (L2), no LDS staging.
//
// The tile tables are the plan's (tiles1 / tiles2: group g owns tiles
// [t[g], t[g+1]), routed groups first, the shared expert last) for 32-row
// tiles of 32 H columns (gate/up) and of 64 output columns (down). Inside a
// group, m is fastest.
#include "device_common.h"
#include "internal.h"

namespace dsmoe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRowsF32 = 32;   // rows per tile (one wave)
constexpr int kColsF32a = 32;  // H columns per gate/up tile
constexpr int kColsF32b = 64;  // output columns per down tile

// Group of a tile: the last g with tiles[g] <= tile (tiles[0] = 0).
__device__ __forceinline__ int group_of_tile(const int32_t* tiles, int ng, int tile) {
  int lo = 0, hi = ng;  // invariant: tiles[lo] <= tile < tiles[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tiles[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Row of the C = A B^T product tile that accumulator register r of lane l
// holds (the lane's column is l % 32).
__device__ __forceinline__ int c_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// acc += A[32 x k] B[32 x k]^T over k = 0 .. K-1 (K a multiple of 8): lane l
// reads row l % 32 of A (a, or null for a row past the tile) and of B, four
// consecutive k at a time; lanes 0-31 take k0 .. k0+3 and lanes 32-63 k0+4
// .. k0+7, one MFMA per pair (k0 + j, k0 + 4 + j), so every product of the
// contraction enters once.
template <int NB>
__device__ __forceinline__ void mma_rows(const float* a, const float* const (&b)[NB], int K,
                                         int lane, f32x16_t (&acc)[NB]) {
  const int kh = 4 * (lane >> 5);
  for (int k0 = 0; k0 < K; k0 += 8) {
    float4 va = a ? *reinterpret_cast<const float4*>(a + k0 + kh) : float4{0.f, 0.f, 0.f, 0.f};
    float4 vb[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n)
      vb[n] = b[n] ? *reinterpret_cast<const float4*>(b[n] + k0 + kh) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(va.x, vb[n].x, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(va.y, vb[n].y, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(va.z, vb[n].z, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(va.w, vb[n].w, acc[n], 0, 0, 0);
    }
  }
}

struct TileF32 {
  int g;             // group (E: the shared expert)
  int64_t row0;      // first row of the group in the H / permuted layout
  int rows;          // rows of the group
  int m, n;          // row tile and column tile inside the group
};

__device__ __forceinline__ TileF32 tile_f32(const FfnArgs& a, const int32_t* tiles, int tile) {
  TileF32 t;
  t.g = group_of_tile(tiles, a.E + 1, tile);
  const bool shared = t.g == a.E;
  t.row0 = shared ? a.TK : a.offsets[t.g];
  t.rows = shared ? static_cast<int>(a.T) : a.offsets[t.g + 1] - a.offsets[t.g];
  const int mt = (t.rows + kRowsF32 - 1) / kRowsF32;
  const int local = tile - tiles[t.g];
  t.n = local / mt;
  t.m = local - t.n * mt;
  return t;
}

// H[row, j] = silu(x_row . Wg[j]) * (x_row . Wu[j]) for one 32 x 32 tile of
// H: the gate columns j and the up columns Ig + j of the group's [2 Ig, d]
// weights, products accumulated in fp32 on the matrix cores.
__global__ __launch_bounds__(64) void ffn1_f32_kernel(FfnArgs a) {
  const int tile = blockIdx.x;
  if (tile >= a.tiles1[a.E + 1]) return;
  const int lane = threadIdx.x;
  const TileF32 t = tile_f32(a, a.tiles1, tile);
  const bool shared = t.g == a.E;
  const int Ig = shared ? a.Is : a.I;
  const float* W = shared ? static_cast<const float*>(a.ws13)
                          : static_cast<const float*>(a.w13) + static_cast<int64_t>(t.g) * 2 * a.I * a.d;
  // this lane's A row (token) and B rows (gate and up columns)
  const int r = t.m * kRowsF32 + (lane & 31);
  const float* arow = nullptr;
  if (r < t.rows) {
    if (shared) {
      arow = static_cast<const float*>(a.x) + static_cast<int64_t>(r) * a.d;
    } else if (a.perm) {
      const int tok = a.perm[t.row0 + r];
      if (tok >= 0 && tok < a.T) arow = static_cast<const float*>(a.x) + static_cast<int64_t>(tok) * a.d;
    } else {
      arow = static_cast<const float*>(a.xperm) + (t.row0 + r) * a.d;
    }
  }
  const int j = t.n * kColsF32a + (lane & 31);
  const float* const b[2] = {j < Ig ? W + static_cast<int64_t>(j) * a.d : nullptr,
                             j < Ig ? W + static_cast<int64_t>(Ig + j) * a.d : nullptr};
  f32x16_t acc[2] = {};
  mma_rows<2>(arow, b, a.d, lane, acc);
  if (j >= Ig) return;
  float* H = static_cast<float*>(a.H);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = t.m * kRowsF32 + c_row(lane, i);
    if (rr < t.rows) H[(t.row0 + rr) * a.ldh + j] = silu_f32(acc[0][i]) * acc[1][i];
  }
}

// y[row, n] = H_row . W2[n] for one 32 x 64 tile of the output: the group's
// [d, Ig] down weights, written to yperm (routed rows) or yshared.
__global__ __launch_bounds__(64) void ffn2_f32_kernel(FfnArgs a) {
  const int tile = blockIdx.x;
  if (tile >= a.tiles2[a.E + 1]) return;
  const int lane = threadIdx.x;
  const TileF32 t = tile_f32(a, a.tiles2, tile);
  const bool shared = t.g == a.E;
  const int Ig = shared ? a.Is : a.I;
  const float* W = shared ? static_cast<const float*>(a.ws2)
                          : static_cast<const float*>(a.w2) + static_cast<int64_t>(t.g) * a.d * a.I;
  const int r = t.m * kRowsF32 + (lane & 31);
  const float* arow =
      r < t.rows ? static_cast<const float*>(a.H) + (t.row0 + r) * a.ldh : nullptr;
  const int n0 = t.n * kColsF32b + (lane & 31);
  const float* const b[2] = {n0 < a.d ? W + static_cast<int64_t>(n0) * Ig : nullptr,
                             n0 + 32 < a.d ? W + static_cast<int64_t>(n0 + 32) * Ig : nullptr};
  f32x16_t acc[2] = {};
  mma_rows<2>(arow, b, Ig, lane, acc);
  float* out = shared ? static_cast<float*>(a.yshared) : static_cast<float*>(a.yperm);
  const int64_t base = shared ? 0 : t.row0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = n0 + 32 * h;
    if (n >= a.d) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = t.m * kRowsF32 + c_row(lane, i);
      if (rr < t.rows) out[(base + rr) * a.d + n] = acc[h][i];
    }
  }
}

}  // namespace

GemmTiling tiling_f32() {
  GemmTiling t{};
  t.bm1 = kRowsF32;
  t.bnh1 = kColsF32a;
  t.bm2 = kRowsF32;
  t.bn2 = kColsF32b;
  t.variant = 2;
  return t;
}

hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  const int64_t rows = a.TK + (a.Is > 0 ? a.T : 0);
  if (rows == 0) return hipSuccess;
  // upper bounds of the plan's tile counts: every group's last row tile may
  // be partial
  const int ldh = a.ldh;
  const int64_t mt = rows / kRowsF32 + a.E + 1;
  const int64_t n1 = mt * ((ldh + kColsF32a - 1) / kColsF32a);
  const int64_t n2 = mt * ((a.d + kColsF32b - 1) / kColsF32b);
  hipLaunchKernelGGL(ffn1_f32_kernel, dim3(static_cast<unsigned>(n1)), dim3(64), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(ffn2_f32_kernel, dim3(static_cast<unsigned>(n2)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsmoe
