// Bandwidth-bound kernels: gated combine, bias update, FP8 quantizers.
#pragma clang fp contract(off)

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace dsmoe {

namespace {

// y[t] = y_shared[t] + sum_k gate[t,k] * y_perm[inv[t,k]]: the shared expert
// is ungated and sees every token (mhpq.cn "DeepSeek-V3 高效训练关键技术全景
// 解析" §1.1); routed outputs weighted by the normalized gates (kaiyunto.com
// DeepSeek-V3 walkthrough). One workgroup per token with one 16-byte chunk of
// the row per thread (d / 8 threads up to 1024: all K + 1 loads of a thread
// are in flight together), fp32 accumulation in slot order. KT > 0 fixes K
// at compile time so the K gathered rows of a chunk are all loaded before
// the (in-order) FMAs.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(w[q] << 16);
    f[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
}

template <int KT, bool OUT_F32>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(const uint16_t* __restrict__ yperm,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ gate,
                                                           const uint16_t* __restrict__ yshared,
                                                           void* __restrict__ y, int K_rt, int d) {
  const int K = KT > 0 ? KT : K_rt;
  const int64_t t = blockIdx.x;
  const int nch = d / 8;
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    float acc[8];
    if (yshared) {
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(yshared + t * d + c * 8), acc);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    }
    if constexpr (KT > 0) {
      uint4 v[KT];
#pragma unroll
      for (int k = 0; k < KT; ++k)
        v[k] = *reinterpret_cast<const uint4*>(yperm + static_cast<int64_t>(inv[t * KT + k]) * d +
                                               c * 8);
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const float g = gate[t * KT + k];
        float f[8];
        bf16x8_to_f32(v[k], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(g, f[q], acc[q]);
      }
    } else {
      for (int k = 0; k < K; ++k) {
        const float g = gate[t * K + k];
        float f[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(
                          yperm + static_cast<int64_t>(inv[t * K + k]) * d + c * 8), f);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(g, f[q], acc[q]);
      }
    }
    if constexpr (OUT_F32) {
      float4* yo = reinterpret_cast<float4*>(static_cast<float*>(y) + t * d + c * 8);
      yo[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      yo[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + t * d + c * 8) = o;
    }
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ yperm,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gate,
                                                          const float* __restrict__ yshared,
                                                          void* __restrict__ y, int K, int d) {
  const int64_t t = blockIdx.x;
  const int nch = d / 4;
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    float4 acc = yshared ? *reinterpret_cast<const float4*>(yshared + t * d + c * 4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
      const float g = gate[t * K + k];
      const int64_t row = inv[t * K + k];
      const float4 v = *reinterpret_cast<const float4*>(yperm + row * d + c * 4);
      acc.x = __builtin_fmaf(g, v.x, acc.x);
      acc.y = __builtin_fmaf(g, v.y, acc.y);
      acc.z = __builtin_fmaf(g, v.z, acc.z);
      acc.w = __builtin_fmaf(g, v.w, acc.w);
    }
    if constexpr (OUT_BF16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + t * d + c * 4) =
          make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(y) + t * d + c * 4) = acc;
  }
}

// b[e] -= gamma when expert e is overloaded (counts*E > T*K), += gamma when
// underloaded, unchanged at exactly the balanced load (kaiyunto.com
// DeepSeek-V3 walkthrough: bias update speed gamma; mhpq.cn §1.2: every step).
__global__ void bias_update_kernel(const int32_t* __restrict__ counts, float gamma,
                                   float* __restrict__ bias, int E, int64_t total) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t load = static_cast<int64_t>(counts[e]) * E;
  if (load > total) bias[e] = bias[e] - gamma;
  else if (load < total) bias[e] = bias[e] + gamma;
}

// Max-abs scaling of one group (mhpq.cn §4.1, online max-abs; gkm0120.cn
// notes Q8, 1x128 tiles / 128x128 blocks): scale = amax/max and codes of
// v * (max/amax), max the format's largest value (448 for E4M3, 57344 for
// E5M2); an all-zero group gets scale 1 and zero codes.
template <int FMT = 0>
__device__ __forceinline__ void quant_params(float amax, float& inv, float& scale) {
  if (amax == 0.0f) {
    inv = 0.0f;
    scale = 1.0f;
  } else {
    inv = Fp8Fmt<FMT>::kMax / amax;
    scale = amax / Fp8Fmt<FMT>::kMax;
  }
}

// Eight consecutive elements src[i .. i+8) as fp32 (i a multiple of 8; one
// 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const void* src, int dtype, int64_t i, float (&v)[8]) {
  if (dtype == 1) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Codes of v * inv for eight values (all zero when the group is all zero).
template <int FMT = 0>
__device__ __forceinline__ uint2 encode8(const float (&v)[8], float amax, float inv) {
  if (amax == 0.0f) return make_uint2(0u, 0u);
  return make_uint2(Fp8Fmt<FMT>::pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                    Fp8Fmt<FMT>::pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv));
}

// One workgroup (256 threads) per 128x128 block: 16 lanes cover one block row
// with 8 elements each (coalesced 16-byte loads), 8 rows per thread.
__global__ __launch_bounds__(256) void quant_blocks_kernel(const void* __restrict__ src,
                                                           int dtype, int rows, int cols,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
  __shared__ float red[4];
  const int rb = rows / 128, cb = cols / 128;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / (static_cast<int64_t>(rb) * cb);
  const int bi = static_cast<int>((blk / cb) % rb), bj = static_cast<int>(blk % cb);
  const int tid = threadIdx.x;
  const int c = tid & 15, r0 = tid >> 4;
  const int64_t base = mat * rows * static_cast<int64_t>(cols) +
                       static_cast<int64_t>(bi * 128 + r0) * cols + bj * 128 + c * 8;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    load8(src, dtype, base + static_cast<int64_t>(16 * i) * cols, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  }
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float inv, sc;
  quant_params(amax, inv, sc);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(q + base + static_cast<int64_t>(16 * i) * cols) =
        encode8(v[i], amax, inv);
  if (tid == 0) scale[blk] = sc;
}

// 16 lanes per 1x128 tile (8 elements each, 16-byte loads), 16 tiles per
// workgroup; rows gathered through perm when given. FMT: 0 E4M3, 1 E5M2.
template <int FMT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, int dtype,
                                                         const int32_t* __restrict__ perm,
                                                         int64_t n, int cols,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale, bool kmajor) {
  const int l16 = threadIdx.x & 15;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int tpr = cols / 128;
  const bool valid = tile < n * tpr;  // lanes stay for the shuffles
  float v[8];
  float amax = 0.0f;
  int64_t base = 0;
  int64_t row = 0;
  int tc = 0;
  if (valid) {
    row = tile / tpr;
    tc = static_cast<int>(tile % tpr);
    const int64_t srow = perm ? static_cast<int64_t>(perm[row]) : row;
    base = row * cols + tc * 128 + l16 * 8;
    load8(src, dtype, srow * cols + tc * 128 + l16 * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  // max over the tile's 16 lanes (xor of the low four lane bits)
  for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (!valid) return;
  float inv, sc;
  quant_params<FMT>(amax, inv, sc);
  *reinterpret_cast<uint2*>(q + base) = encode8<FMT>(v, amax, inv);
  if (l16 == 0) scale[kmajor ? tc * n + row : tile] = sc;
}

}  // namespace

hipError_t launch_combine(const void* yperm, const int32_t* inv, const float* gate,
                          const void* yshared, void* y, int64_t T, int K, int d, int io_dtype,
                          int out_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (io_dtype == 1) {
    const auto* yp = static_cast<const uint16_t*>(yperm);
    const auto* ys = static_cast<const uint16_t*>(yshared);
    int nthr = ((d / 8 + 63) / 64) * 64;
    if (nthr > 1024) nthr = 1024;
    const dim3 grid(static_cast<unsigned>(T)), block(static_cast<unsigned>(nthr));
    auto go = [&](auto out_f32) {
      constexpr bool F = decltype(out_f32)::value;
      if (K == 8)
        hipLaunchKernelGGL((combine_bf16_kernel<8, F>), grid, block, 0, s, yp, inv, gate, ys, y, K,
                           d);
      else if (K == 6)
        hipLaunchKernelGGL((combine_bf16_kernel<6, F>), grid, block, 0, s, yp, inv, gate, ys, y, K,
                           d);
      else
        hipLaunchKernelGGL((combine_bf16_kernel<0, F>), grid, block, 0, s, yp, inv, gate, ys, y, K,
                           d);
    };
    if (out_dtype == 0)
      go(std::true_type{});
    else
      go(std::false_type{});
  } else {
    const auto* yp = static_cast<const float*>(yperm);
    const auto* ys = static_cast<const float*>(yshared);
    if (out_dtype == 1)
      hipLaunchKernelGGL(combine_f32_kernel<true>, dim3(static_cast<unsigned>(T)), dim3(256), 0, s,
                         yp, inv, gate, ys, y, K, d);
    else
      hipLaunchKernelGGL(combine_f32_kernel<false>, dim3(static_cast<unsigned>(T)), dim3(256), 0,
                         s, yp, inv, gate, ys, y, K, d);
  }
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, float gamma, float* bias, int E, int64_t T,
                              int K, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, s, counts, gamma,
                     bias, E, T * K);
  return hipGetLastError();
}

hipError_t launch_quant_blocks(const void* src, int src_dtype, int64_t n_mats, int rows, int cols,
                               uint8_t* q, float* scale, hipStream_t s) {
  const int64_t blocks = n_mats * (rows / 128) * static_cast<int64_t>(cols / 128);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_blocks_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src,
                     src_dtype, rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* src, int src_dtype, const int32_t* perm, int64_t n,
                             int cols, uint8_t* q, float* scale, hipStream_t s, int fmt,
                             bool kmajor) {
  const int64_t tiles = n * (cols / 128);
  if (tiles == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((tiles + 15) / 16)), block(256);
  if (fmt == 1)
    hipLaunchKernelGGL(quant_rows_kernel<1>, grid, block, 0, s, src, src_dtype, perm, n, cols, q,
                       scale, kmajor);
  else
    hipLaunchKernelGGL(quant_rows_kernel<0>, grid, block, 0, s, src, src_dtype, perm, n, cols, q,
                       scale, kmajor);
  return hipGetLastError();
}

}  // namespace dsmoe
