// Routing: sigmoid affinities, selection bias, group limit, top-K, gates,
// per-expert counts and near-tie count (kaiyunto.com DeepSeek-V3 walkthrough,
// DeepSeekMoE paragraph; gkm0120.cn notes Q3; mhpq.cn "DeepSeek-V3 高效训练
// 关键技术全景解析" §1.2 and §3.1).
//
// Every routing decision is a fixed sequence of IEEE fp32 operations with no
// contraction, so the result is reproducible bit for bit from the logits.
// This file is compiled with -ffp-contract=off in addition to the pragma.
#pragma clang fp contract(off)

#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "route_token.h"
#include "sigmoid_ieee.h"

namespace dsmoe {

namespace {

// partial[i] = ((partial[i] + partial[n + i]) + ...) + partial[(S-1) n + i]:
// the split-K partial sums of the router product added in split order, one
// thread per logit. Used when there are many splits (small T), where the
// routing kernel's one wave per token would add them with little parallelism;
// the order, and so every bit, is the routing kernel's own.
__global__ __launch_bounds__(256) void sum_partials_kernel(float* __restrict__ partial, int splits,
                                                           int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float u = partial[i];
  // loads in groups of eight so they are in flight together; adds in order
  for (int q0 = 1; q0 < splits; q0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = q0 + j < splits ? partial[static_cast<int64_t>(q0 + j) * n + i] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q0 + j < splits) u = u + v[j];
  }
  partial[i] = u;
}

// Router for small batches (T <= kSmallRouterT, bf16 activations): the fp32
// weights are read once and multiplied on the VALU, fp32 FMA per term (one
// rounding per term, as with the exact bf16-split products added in fp32).
// Block b handles experts [b*EPB, (b+1)*EPB) for all tokens. Each thread
// owns the 4-element k groups tid + 512 q of d; its weight groups stay in
// registers and the activation groups of eight tokens are loaded together,
// so a pass waits for memory once. The per-thread partial dot products are
// reduced in a fixed order (shuffle tree, then the eight waves in order), so
// every run gives the same bits. Block 0 also clears the per-expert counts
// and the near-tie count that the routing kernel adds to.
constexpr int kSmallEPB = 2;       // experts per block
constexpr int kSmallThreads = 512;
constexpr int kSmallKPT = 4;       // 4-element k groups per thread per chunk
constexpr int kSmallMaxT = 32;

__global__ __launch_bounds__(kSmallThreads) void router_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w, int T, int d, int E,
    float* __restrict__ out, int32_t* __restrict__ counts, int32_t* __restrict__ near_tie) {
  constexpr int NW = kSmallThreads / 64;
  __shared__ float red[NW][kSmallEPB * kSmallMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kSmallThreads) counts[e] = 0;
    if (tid == 0 && near_tie) *near_tie = 0;
  }
  const int e0 = blockIdx.x * kSmallEPB;
  const int d4 = d >> 2;
  float acc[kSmallEPB][kSmallMaxT];
#pragma unroll
  for (int i = 0; i < kSmallEPB; ++i)
#pragma unroll
    for (int t = 0; t < kSmallMaxT; ++t) acc[i][t] = 0.0f;
  for (int kc = 0; kc < d4; kc += kSmallThreads * kSmallKPT) {
    float4 wv[kSmallEPB][kSmallKPT];
#pragma unroll
    for (int i = 0; i < kSmallEPB; ++i)
#pragma unroll
      for (int q = 0; q < kSmallKPT; ++q) {
        const int k4 = kc + tid + kSmallThreads * q;
        wv[i][q] = (e0 + i < E && k4 < d4)
                       ? reinterpret_cast<const float4*>(w + static_cast<int64_t>(e0 + i) * d)[k4]
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int t0 = 0; t0 < kSmallMaxT; t0 += 8) {
      if (t0 >= T) continue;
      uint2 xv[8][kSmallKPT];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int q = 0; q < kSmallKPT; ++q) {
          const int k4 = kc + tid + kSmallThreads * q;
          xv[j][q] = (t0 + j < T && k4 < d4)
                         ? reinterpret_cast<const uint2*>(x + static_cast<int64_t>(t0 + j) * d)[k4]
                         : make_uint2(0u, 0u);
        }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int q = 0; q < kSmallKPT; ++q) {
          const float x0 = bf16_to_f32(static_cast<uint16_t>(xv[j][q].x & 0xFFFFu));
          const float x1 = bf16_to_f32(static_cast<uint16_t>(xv[j][q].x >> 16));
          const float x2 = bf16_to_f32(static_cast<uint16_t>(xv[j][q].y & 0xFFFFu));
          const float x3 = bf16_to_f32(static_cast<uint16_t>(xv[j][q].y >> 16));
#pragma unroll
          for (int i = 0; i < kSmallEPB; ++i) {
            float v = acc[i][t0 + j];
            v = __builtin_fmaf(x0, wv[i][q].x, v);
            v = __builtin_fmaf(x1, wv[i][q].y, v);
            v = __builtin_fmaf(x2, wv[i][q].z, v);
            v = __builtin_fmaf(x3, wv[i][q].w, v);
            acc[i][t0 + j] = v;
          }
        }
    }
  }
  // fixed-order reduction. Reduce-scatter butterfly over the wave: at the
  // step with lane bit o, a lane keeps the half of its values whose index has
  // that bit equal to its own, adds the partner's copy of that half, and
  // sends the other half; after six steps lane l holds the wave's sum for
  // value index l = (expert in block) * 32 + token. Then the waves in order.
  static_assert(kSmallEPB * kSmallMaxT == 64, "one value per lane after the butterfly");
  float v[64];
#pragma unroll
  for (int i = 0; i < kSmallEPB; ++i)
#pragma unroll
    for (int t = 0; t < kSmallMaxT; ++t) v[i * kSmallMaxT + t] = acc[i][t];
#pragma unroll
  for (int n = 64, o = 32; o >= 1; n >>= 1, o >>= 1) {
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float keep = upper ? v[i + n / 2] : v[i];
      const float send = upper ? v[i] : v[i + n / 2];
      v[i] = keep + __shfl_xor(send, o, 64);
    }
  }
  red[wave][lane] = v[0];
  __syncthreads();
  if (tid < 64) {
    const int i = tid / kSmallMaxT, t = tid % kSmallMaxT;
    if (t < T && e0 + i < E) {
      float r = red[0][tid];
#pragma unroll
      for (int q = 1; q < NW; ++q) r = r + red[q][tid];
      out[static_cast<int64_t>(t) * E + e0 + i] = r;
    }
  }
}

constexpr int kTokPerBlock = 4;  // one wave per token

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ partial, int splits,
                                                    float* __restrict__ logits_out,
                                                    const float* __restrict__ bias, RouteParams p,
                                                    int32_t* __restrict__ idx_out,
                                                    float* __restrict__ gate_out,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ near_tie) {
  __shared__ float c_lds[kTokPerBlock][kMaxE];
  __shared__ float s_lds[kTokPerBlock][kMaxE];
  __shared__ int hist[kMaxE];
  __shared__ int ntie;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int E = p.E;
  for (int e = tid; e < E; e += blockDim.x) hist[e] = 0;
  if (tid == 0) ntie = 0;
  __syncthreads();

  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kTokPerBlock; base < p.T;
       base += static_cast<int64_t>(gridDim.x) * kTokPerBlock) {
    const int64_t t = base + wave;
    if (t >= p.T) break;
    // the token's logits: the split-K partials (fewer than eight), all loads
    // in flight together, then added in split order
    float pv[EPL][8];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      const size_t off = static_cast<size_t>(t) * E + e;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        pv[j][q] = (e < E && q < splits) ? partial[static_cast<size_t>(q) * p.T * E + off] : 0.0f;
    }
    float u[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      float v = pv[j][0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (q < splits) v = v + pv[j][q];
      u[j] = v;
      if (logits_out && e < E) logits_out[static_cast<size_t>(t) * E + e] = v;
    }
    route_token<EPL>(u, t, bias, p, c_lds[wave], s_lds[wave], lane, idx_out, gate_out, hist,
                     &ntie);
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
  if (tid == 0 && ntie && near_tie) atomicAdd(near_tie, ntie);
}

// fp32 activations: plain fp32 dot products, one wave per (token, expert).
// Lane l takes the 4-element pieces l, l + 64, ... of the contraction (d is
// a multiple of 64, rows 16-byte aligned), and a butterfly over the wave adds
// the 64 partial sums in a fixed order.
constexpr int kRouterF32Waves = 4;  // waves (dot products) per workgroup
__global__ __launch_bounds__(64 * kRouterF32Waves) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, int64_t T, int d, int E,
    float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kRouterF32Waves + (threadIdx.x >> 6);
  if (i >= T * E) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int64_t t = i / E;
  const int e = static_cast<int>(i % E);
  const float4* xr = reinterpret_cast<const float4*>(x + t * d);
  const float4* wr = reinterpret_cast<const float4*>(w + static_cast<int64_t>(e) * d);
  float acc = 0.0f;
  for (int k = lane; k < d / 4; k += 64) {
    const float4 a = xr[k], b = wr[k];
    acc = __builtin_fmaf(a.x, b.x, acc);
    acc = __builtin_fmaf(a.y, b.y, acc);
    acc = __builtin_fmaf(a.z, b.z, acc);
    acc = __builtin_fmaf(a.w, b.w, acc);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (lane == 0) out[i] = acc;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n,
                     v);
  return hipGetLastError();
}

hipError_t launch_router_f32(const float* x, const float* w, int64_t T, int d, int E, float* out,
                             hipStream_t s) {
  const int64_t n = T * E;
  if (n == 0) return hipSuccess;
  if (d % 64) return hipErrorInvalidValue;
  const int64_t blocks = (n + kRouterF32Waves - 1) / kRouterF32Waves;
  hipLaunchKernelGGL(router_f32_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * kRouterF32Waves), 0, s, x, w, T, d, E, out);
  return hipGetLastError();
}

hipError_t launch_router_small(const void* x, const float* w, int64_t T, int d, int E, float* out,
                               int32_t* counts, int32_t* near_tie, hipStream_t s) {
  const int blocks = (E + kSmallEPB - 1) / kSmallEPB;
  static_assert(kSmallRouterT <= kSmallMaxT, "the small router holds all tokens in registers");
  hipLaunchKernelGGL(router_small_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kSmallThreads), 0, s,
                     static_cast<const uint16_t*>(x), w, static_cast<int>(T), d, E, out, counts,
                     near_tie);
  return hipGetLastError();
}

hipError_t launch_sum_partials(float* partial, int splits, int64_t n, hipStream_t s) {
  if (n == 0 || splits <= 1) return hipSuccess;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, partial, splits, n);
  return hipGetLastError();
}

hipError_t launch_route(const float* partial, int splits, float* logits_out, const float* bias,
                        const RouteParams& p, int32_t* idx, float* gate, int32_t* counts,
                        int32_t* near_tie, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (splits < 1 || splits > 8 || p.E > kMaxE) return hipErrorInvalidValue;
  int64_t blocks = (p.T + kTokPerBlock - 1) / kTokPerBlock;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int epl = (p.E + kWave - 1) / kWave;
  if (epl <= 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, partial, splits, logits_out, bias, p,
                       idx, gate, counts, near_tie);
  else if (epl <= 2)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, partial, splits, logits_out, bias, p,
                       idx, gate, counts, near_tie);
  else if (epl <= 4)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, partial, splits, logits_out, bias, p,
                       idx, gate, counts, near_tie);
  else
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, partial, splits, logits_out, bias, p,
                       idx, gate, counts, near_tie);
  return hipGetLastError();
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace dsmoe
