// Achievable-peak microbenchmarks of one MI355X (gfx950), the second column
// next to the published peaks in the benchmark: a streaming HBM read, and
// MFMA issue rates for bf16 (v_mfma_f32_32x32x16_bf16) and FP8
// (v_mfma_scale_f32_32x32x64_f8f6f4) with operands in registers. Built into
// libdsmoe_microbench.so, loaded by bench.py only; not part of the layer's
// C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "tile_schedule.h"

namespace {

using dsmoe::dma16;
using dsmoe::dma16_nt;
using dsmoe::i32x4_t;
using dsmoe::lds_addr;
using dsmoe::rsrc4;
using dsmoe::vm_wait;

// The layer's load path: 16-byte buffer loads straight into LDS (one 1 KB
// piece per wave and instruction; NT: non-temporal like the decode GEMMs'
// weight loads, else the default policy of the prefill GEMMs), each wave
// cycling over 8 slots of its own 8 KB LDS ring, at most 24 loads in flight;
// workgroup b reads pieces b, b + nb, ... of the buffer (bytes < 2^31). Five
// workgroups per CU fill its LDS and read fastest.
template <bool NT>
__global__ __launch_bounds__(256) void hbm_dma_kernel(const void* src, uint32_t bytes) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][8][1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const i32x4_t r = rsrc4(src, bytes);
  const uint32_t pieces = bytes / 1024u;
  const uint32_t nw = gridDim.x * 4u;
  uint32_t p = blockIdx.x * 4u + wave;
  int slot = 0;
  for (; p + 7 * nw < pieces; p += 8 * nw) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(&ring[wave][slot][0]));
      if constexpr (NT)
        dma16_nt(r, (p + u * nw) * 1024u + lane * 16u, dst);
      else
        dma16(r, (p + u * nw) * 1024u + lane * 16u, dst);
      slot = (slot + 1) & 7;
    }
    vm_wait<16>();
  }
  vm_wait<0>();
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Every thread reads 16-byte chunks in a grid-stride loop (eight in flight,
// non-temporal) and folds them into one word, written out so that no load is
// dead.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4_t* __restrict__ src,
                                                       int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = NT ? __builtin_nontemporal_load(&src[i + u * stride]) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// Every thread writes 16-byte chunks (VEC) or 4-byte words in a grid-stride
// loop; NT: non-temporal stores. The written values depend on the index so
// nothing is constant-folded.
template <bool NT, bool VEC>
__global__ __launch_bounds__(256) void hbm_write_kernel(uint32_t* __restrict__ dst, int64_t n32) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if constexpr (VEC) {
    u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
    const int64_t n = n32 / 4;
    for (int64_t i = i0; i < n; i += stride) {
      const uint32_t v = static_cast<uint32_t>(i);
      const u32x4_t w = {v, v + 1u, v + 2u, v + 3u};
      if constexpr (NT)
        __builtin_nontemporal_store(w, &d[i]);
      else
        d[i] = w;
    }
  } else {
    for (int64_t i = i0; i < n32; i += stride) {
      if constexpr (NT)
        __builtin_nontemporal_store(static_cast<uint32_t>(i), &dst[i]);
      else
        dst[i] = static_cast<uint32_t>(i);
    }
  }
}

// Eight independent accumulators per wave, so the matrix core never waits
// on a result; the operands change every iteration so nothing is hoisted.
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(0.001f * (lane + j));
    b[j] = static_cast<__bf16>(0.002f * (lane - j));
  }
  f32x16_t acc[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
    a[0] = static_cast<__bf16>(static_cast<float>(a[0]) + 1.0f);
  }
  float s = 0.0f;
  for (int u = 0; u < 8; ++u)
    for (int r = 0; r < 16; ++r) s += acc[u][r];
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_fp8_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  i32x8_t a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = 0x38383838 + lane + j;
    b[j] = 0x30303030 + lane - j;
  }
  f32x16_t acc[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[u], 0, 0, 0, 127, 0, 127);
    a[0] ^= 1;
  }
  float s = 0.0f;
  for (int u = 0; u < 8; ++u)
    for (int r = 0; r < 16; ++r) s += acc[u][r];
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// The same over the LDS-DMA load path; bytes a multiple of 1 KB, < 2^31.
// Non-temporal loads; dsmoe_mb_hbm_dma_default: the default cache policy.
int dsmoe_mb_hbm_dma(const void* src, int64_t bytes, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(hbm_dma_kernel<true>, dim3(blocks), dim3(256), 0, s, src,
                     static_cast<uint32_t>(bytes));
  return hipGetLastError();
}
int dsmoe_mb_hbm_dma_default(const void* src, int64_t bytes, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(hbm_dma_kernel<false>, dim3(blocks), dim3(256), 0, s, src,
                     static_cast<uint32_t>(bytes));
  return hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from src with `blocks` workgroups of 256
// threads; sink holds blocks * 256 words. Returns a hipError_t.
int dsmoe_mb_hbm_read(const void* src, int64_t bytes, int blocks, void* sink, hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(blocks), dim3(256), 0, s,
                     static_cast<const u32x4_t*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}
// The same with the default cache policy.
int dsmoe_mb_hbm_read_default(const void* src, int64_t bytes, int blocks, void* sink,
                              hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(blocks), dim3(256), 0, s,
                     static_cast<const u32x4_t*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

// Writes `bytes` (a multiple of 16) to dst with `blocks` workgroups of 256
// threads: mode bit 0 = non-temporal stores, bit 1 = 16-byte stores (else
// 4-byte words). Returns a hipError_t.
int dsmoe_mb_hbm_write(void* dst, int64_t bytes, int blocks, int mode, hipStream_t s) {
  uint32_t* d = static_cast<uint32_t*>(dst);
  const int64_t n32 = bytes / 4;
  switch (mode & 3) {
    case 0: hipLaunchKernelGGL((hbm_write_kernel<false, false>), dim3(blocks), dim3(256), 0, s, d, n32); break;
    case 1: hipLaunchKernelGGL((hbm_write_kernel<true, false>), dim3(blocks), dim3(256), 0, s, d, n32); break;
    case 2: hipLaunchKernelGGL((hbm_write_kernel<false, true>), dim3(blocks), dim3(256), 0, s, d, n32); break;
    default: hipLaunchKernelGGL((hbm_write_kernel<true, true>), dim3(blocks), dim3(256), 0, s, d, n32); break;
  }
  return hipGetLastError();
}

// `blocks` workgroups of 4 waves, each wave issuing iters * 8 MFMAs of
// 32x32x16 bf16 (32768 flops each) / 32x32x64 fp8 (131072 flops each); sink
// holds blocks * 256 floats.
int dsmoe_mb_mfma(int fp8, int iters, int blocks, void* sink, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL(mfma_fp8_kernel, dim3(blocks), dim3(256), 0, s, iters,
                       static_cast<float*>(sink));
  else
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, s, iters,
                       static_cast<float*>(sink));
  return hipGetLastError();
}

}  // extern "C"
