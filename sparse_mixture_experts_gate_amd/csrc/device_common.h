// Device helpers shared by the HIP kernels of the library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Four bf16 values as one 8-byte word.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// silu(z) = z * sigmoid(z) for the expert activations (tolerance-checked).
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// One E4M3FN code from an fp32 value already scaled into [-448, 448]: clamp
// (saturation), then the hardware conversion, which rounds to nearest even.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Four E5M2 codes (the backward's gradient format) from fp32 values already
// scaled into [-57344, 57344]: clamp (saturation), then the hardware
// conversion, which rounds to nearest even.
__device__ __forceinline__ uint32_t e5m2_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -57344.0f), 57344.0f);
  b = fminf(fmaxf(b, -57344.0f), 57344.0f);
  c = fminf(fmaxf(c, -57344.0f), 57344.0f);
  d = fminf(fmaxf(d, -57344.0f), 57344.0f);
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// FP8 formats of the layer: E4M3 (forward operands, weights, activations)
// and E5M2 (backward gradients); the largest finite value of each.
template <int FMT>
struct Fp8Fmt;
template <>
struct Fp8Fmt<0> {
  static constexpr float kMax = 448.0f;
  __device__ static uint32_t pack4(float a, float b, float c, float d) {
    return e4m3_pack4(a, b, c, d);
  }
};
template <>
struct Fp8Fmt<1> {
  static constexpr float kMax = 57344.0f;
  __device__ static uint32_t pack4(float a, float b, float c, float d) {
    return e5m2_pack4(a, b, c, d);
  }
};

// Maps a physical workgroup id to a logical one so that logically adjacent
// workgroups run on the same XCD (workgroups are dealt round-robin over the
// 8 XCDs, each with its own L2). Requires gridDim.x % 8 == 0.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

// One tile per workgroup: the blocks of XCD x (x, x + 8, x + 16, ...) take
// tiles [x per, (x + 1) per), per = ceil(total / 8), in order, so the tiles an
// XCD runs at a time are a contiguous window of the tile order (tiles that
// share an operand slab stay together however long each takes). -1: no tile.
__device__ __forceinline__ int xcd_single_tile(int b, int total) {
  const int per = (total + 7) / 8, slot = b >> 3;
  const int t = (b & 7) * per + slot;
  return (slot < per && t < total) ? t : -1;
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace dsmoe
