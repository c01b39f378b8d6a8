// fp32 sigmoid of the router logits (affinity scores are sigmoids of the
// logits: kaiyunto.com DeepSeek-V3 walkthrough, DeepSeekMoE paragraph), from
// IEEE + - * /, rint and ldexp only, without contraction, so that every
// kernel that needs a score recomputes the same bits.
#pragma once

#include "device_common.h"

namespace dsmoe {
namespace {

// exp(v) = 2^n exp(r), n = rint(v log2 e), r = v - n ln2 in two pieces
// (Cody-Waite; ln2_hi = 355/512 has 9 significant bits so n*ln2_hi is exact),
// exp(r) from the degree-7 Taylor polynomial, Horner form.
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kLn2Hi = 0x1.63p-1f;
constexpr float kLn2Lo = -0x1.bd0106p-13f;
constexpr float kC0 = 1.0f, kC1 = 1.0f, kC2 = 0x1p-1f, kC3 = 0x1.555556p-3f,
                kC4 = 0x1.555556p-5f, kC5 = 0x1.111112p-7f, kC6 = 0x1.6c16c2p-10f,
                kC7 = 0x1.a01a02p-13f;

__device__ __forceinline__ float sigmoid_ieee(float u) {
#pragma clang fp contract(off)
  const float v = -u;
  if (v > 87.0f) return 0.0f;   // exp(v) would leave the normal range
  if (v < -20.0f) return 1.0f;  // 1 + exp(v) rounds to 1
  const float n = __builtin_rintf(v * kLog2e);
  const float r = (v - n * kLn2Hi) - n * kLn2Lo;
  float p = kC7;
  p = p * r; p = p + kC6;
  p = p * r; p = p + kC5;
  p = p * r; p = p + kC4;
  p = p * r; p = p + kC3;
  p = p * r; p = p + kC2;
  p = p * r; p = p + kC1;
  p = p * r; p = p + kC0;
  const float e = __builtin_ldexpf(p, static_cast<int>(n));
  return 1.0f / (1.0f + e);
}


}  // namespace
}  // namespace dsmoe
