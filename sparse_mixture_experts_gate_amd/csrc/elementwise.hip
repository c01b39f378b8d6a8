// Bandwidth-bound kernels: gated combine, bias update, FP8 quantizers.
#pragma clang fp contract(off)

#include "device_common.h"
#include "internal.h"

namespace dsmoe {

namespace {

// y[t] = y_shared[t] + sum_k gate[t,k] * y_perm[inv[t,k]]: the shared expert
// is ungated and sees every token (mhpq.cn "DeepSeek-V3 高效训练关键技术全景
// 解析" §1.1); routed outputs weighted by the normalized gates (kaiyunto.com
// DeepSeek-V3 walkthrough). One workgroup per token, 16-byte accesses,
// fp32 accumulation in slot order.
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t* __restrict__ yperm,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ gate,
                                                           const uint16_t* __restrict__ yshared,
                                                           uint16_t* __restrict__ y, int K, int d) {
  const int64_t t = blockIdx.x;
  const int nch = d / 8;
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    float acc[8];
    if (yshared) {
      const uint4 v = *reinterpret_cast<const uint4*>(yshared + t * d + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __uint_as_float(w[q] << 16);
        acc[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    }
    for (int k = 0; k < K; ++k) {
      const float g = gate[t * K + k];
      const int64_t row = inv[t * K + k];
      const uint4 v = *reinterpret_cast<const uint4*>(yperm + row * d + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __builtin_fmaf(g, __uint_as_float(w[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(g, __uint_as_float(w[q] & 0xFFFF0000u), acc[2 * q + 1]);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + t * d + c * 8) = o;
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ yperm,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gate,
                                                          const float* __restrict__ yshared,
                                                          float* __restrict__ y, int K, int d) {
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
    *reinterpret_cast<float4*>(y + t * d + c * 4) = acc;
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

__device__ __forceinline__ float load_src(const void* src, int dtype, int64_t i) {
  return dtype == 1 ? bf16_to_f32(static_cast<const uint16_t*>(src)[i])
                    : static_cast<const float*>(src)[i];
}

// Max-abs scaling of one group (mhpq.cn §4.1, online max-abs; gkm0120.cn
// notes Q8, 1x128 tiles / 128x128 blocks): scale = amax/448 and codes of
// v * (448/amax); an all-zero group gets scale 1 and zero codes.
__device__ __forceinline__ void quant_params(float amax, float& inv, float& scale) {
  if (amax == 0.0f) {
    inv = 0.0f;
    scale = 1.0f;
  } else {
    inv = 448.0f / amax;
    scale = amax / 448.0f;
  }
}

// One workgroup (256 threads) per 128x128 block; each thread 64 elements.
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
  // thread -> (row, 64-column half) of the block, rows tid/2
  const int r = tid >> 1, c0 = (tid & 1) * 64;
  const int64_t base = mat * rows * static_cast<int64_t>(cols) +
                       static_cast<int64_t>(bi * 128 + r) * cols + bj * 128 + c0;
  float v[64];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    v[j] = load_src(src, dtype, base + j);
    amax = fmaxf(amax, fabsf(v[j]));
  }
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float inv, sc;
  quant_params(amax, inv, sc);
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const uint32_t w = amax == 0.0f ? 0u
                                    : e4m3_pack4(v[j] * inv, v[j + 1] * inv, v[j + 2] * inv,
                                                 v[j + 3] * inv);
    *reinterpret_cast<uint32_t*>(q + base + j) = w;
  }
  if (tid == 0) scale[blk] = sc;
}

// One wave per 1x128 tile; each lane 2 elements.
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, int dtype,
                                                         const int32_t* __restrict__ perm,
                                                         int64_t n, int cols,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int tpr = cols / 128;
  if (tile >= n * tpr) return;
  const int64_t row = tile / tpr;
  const int tc = static_cast<int>(tile % tpr);
  const int64_t srow = perm ? static_cast<int64_t>(perm[row]) : row;
  const int64_t base = row * cols + tc * 128 + lane * 2;
  const int64_t sbase = srow * cols + tc * 128 + lane * 2;
  const float a = load_src(src, dtype, sbase), b = load_src(src, dtype, sbase + 1);
  float amax = fmaxf(fabsf(a), fabsf(b));
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  float inv, sc;
  quant_params(amax, inv, sc);
  const uint32_t w = amax == 0.0f ? 0u : e4m3_pack4(a * inv, b * inv, 0.0f, 0.0f);
  *reinterpret_cast<uint16_t*>(q + base) = static_cast<uint16_t>(w & 0xFFFFu);
  if (lane == 0) scale[tile] = sc;
}

}  // namespace

hipError_t launch_combine(const void* yperm, const int32_t* inv, const float* gate,
                          const void* yshared, void* y, int64_t T, int K, int d, int io_dtype,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (io_dtype == 1)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(yperm), inv, gate,
                       static_cast<const uint16_t*>(yshared), static_cast<uint16_t*>(y), K, d);
  else
    hipLaunchKernelGGL(combine_f32_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, s,
                       static_cast<const float*>(yperm), inv, gate,
                       static_cast<const float*>(yshared), static_cast<float*>(y), K, d);
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
                             int cols, uint8_t* q, float* scale, hipStream_t s) {
  const int64_t tiles = n * (cols / 128);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(static_cast<unsigned>((tiles + 3) / 4)), dim3(256), 0,
                     s, src, src_dtype, perm, n, cols, q, scale);
  return hipGetLastError();
}

}  // namespace dsmoe
