// Routing of one token by one wave: sigmoid affinities, selection bias, group
// limit, top-K, gates, the selection counted into a histogram and the near-tie
// flag (kaiyunto.com DeepSeek-V3 walkthrough, DeepSeekMoE paragraph;
// gkm0120.cn notes Q3; mhpq.cn "DeepSeek-V3 高效训练关键技术全景解析" §1.2 and
// §3.1). Shared by the routing kernel and the router GEMM that routes its own
// tiles. Every decision is a fixed sequence of IEEE fp32 operations without
// contraction, so the result is reproducible bit for bit from the logits.
#pragma once

#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "sigmoid_ieee.h"

namespace dsmoe {
namespace {

constexpr int kMaxE = 512;

// (value desc, index asc) total order; the best candidate wins.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Lane moves within 16-lane rows (DPP; every lane has a source lane).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane l <-> 7 - l within 8
constexpr int kDppMirror = 0x140;     // lane l <-> 15 - l within 16
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// Best (value, index) of the wave in every lane. Each step pairs every lane
// with a lane of a disjoint set that holds the same partial result, and
// keeps the better of the two: quads, 8-lane halves and 16-lane rows by DPP,
// then rows and half-waves by shuffles. better() is a strict order, so the
// result is the unique best whatever the pairing.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  auto step = [&](float ov, int oi) {
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  };
  step(dpp_f<kDppXor1>(v), dpp_i<kDppXor1>(i));
  step(dpp_f<kDppXor2>(v), dpp_i<kDppXor2>(i));
  step(dpp_f<kDppHalfMirror>(v), dpp_i<kDppHalfMirror>(i));
  step(dpp_f<kDppMirror>(v), dpp_i<kDppMirror>(i));
  step(__shfl_xor(v, 16, kWave), __shfl_xor(i, 16, kWave));
  step(__shfl_xor(v, 32, kWave), __shfl_xor(i, 32, kWave));
}

// Top two (with multiplicity) of the union of two disjoint sets' top twos.
__device__ __forceinline__ void merge_top2(float& a0, float& a1, float b0, float b1) {
  const float hi = fmaxf(a0, b0), lo = fminf(a0, b0);
  a1 = fmaxf(lo, fmaxf(a1, b1));
  a0 = hi;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// values (the wave's rows are private to it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Routes token t from its fp32 logits: lane l holds the logit of expert
// l + 64 j in u[j] (entries of experts >= E are ignored). c_row / s_row: this
// wave's LDS rows of at least E floats (biased and unbiased scores). Writes
// the token's K expert ids (slots in descending biased score) and gates,
// adds the selected experts to hist and a near tie to *ntie (both LDS).
template <int EPL>
__device__ __forceinline__ void route_token(const float (&u)[EPL], int64_t t,
                                            const float* __restrict__ bias, const RouteParams& p,
                                            float* c_row, float* s_row, int lane,
                                            int32_t* __restrict__ idx_out,
                                            float* __restrict__ gate_out, int* hist, int* ntie) {
#pragma clang fp contract(off)
  const int E = p.E, K = p.K, G = p.G, M = p.M;
  const int GS = E / G;
  float s[EPL], c[EPL];
  bool taken[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + kWave * j;
    taken[j] = false;
    s[j] = 0.0f;
    c[j] = -INFINITY;
    if (e < E) {
      s[j] = sigmoid_ieee(u[j]);
      c[j] = s[j] + bias[e];
      c_row[e] = c[j];
      s_row[e] = s[j];
    }
  }
  wave_lds_sync();

  bool tie = false;
  uint64_t allowed = ~0ull;  // bit g: group g eligible
  if (G > 1) {
    // group score: fp32 sum of the group's topn best biased scores, largest first
    float gsc = -INFINITY;
    if (GS == 32 && p.topn <= 2) {
      // groups of 32 are half-waves: expert lane + 64 j is in group
      // 2 j + lane / 32, so each half-wave reduces its top two in registers
      float gs[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        float t0 = c[j], t1 = -INFINITY;
        merge_top2(t0, t1, dpp_f<kDppXor1>(t0), dpp_f<kDppXor1>(t1));
        merge_top2(t0, t1, dpp_f<kDppXor2>(t0), dpp_f<kDppXor2>(t1));
        merge_top2(t0, t1, dpp_f<kDppHalfMirror>(t0), dpp_f<kDppHalfMirror>(t1));
        merge_top2(t0, t1, dpp_f<kDppMirror>(t0), dpp_f<kDppMirror>(t1));
        merge_top2(t0, t1, __shfl_xor(t0, 16, kWave), __shfl_xor(t1, 16, kWave));
        gs[j] = p.topn == 2 ? t0 + t1 : t0;
      }
      // lane g < G collects group g = 2 (g / 2) + g % 2 from its half-wave
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const float v = __shfl(gs[j], (lane & 1) * 32, kWave);
        if ((lane >> 1) == j && lane < G) gsc = v;
      }
    } else if (lane < G && p.topn <= 2) {
      // the two best (or the best) of the group in two registers
      float t0 = -INFINITY, t1 = -INFINITY;
      for (int i = 0; i < GS; ++i) {
        const float v = c_row[lane * GS + i];
        if (v > t0) { t1 = t0; t0 = v; }
        else if (v > t1) { t1 = v; }
      }
      gsc = p.topn == 2 ? t0 + t1 : t0;
    } else if (lane < G) {
      float top[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) top[q] = -INFINITY;
      for (int i = 0; i < GS; ++i) {
        float v = c_row[lane * GS + i];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (q < p.topn && v > top[q]) { const float tmp = top[q]; top[q] = v; v = tmp; }
        }
      }
      gsc = top[0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (q < p.topn) gsc = gsc + top[q];
    }
    allowed = 0;
    bool picked = false;
    float last = 0.0f;
    for (int q = 0; q < M; ++q) {
      float bv = (lane < G && !picked) ? gsc : -INFINITY;
      int bi = (lane < G && !picked) ? lane : 0x7fffffff;
      wave_argmax(bv, bi);
      allowed |= 1ull << bi;
      if (lane == bi) picked = true;
      last = bv;
    }
    if (G > M) {
      float bv = (lane < G && !picked) ? gsc : -INFINITY;
      int bi = (lane < G && !picked) ? lane : 0x7fffffff;
      wave_argmax(bv, bi);
      if (last - bv <= p.eps) tie = true;
    }
  }

  bool elig[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + kWave * j;
    elig[j] = e < E && ((allowed >> (e / GS)) & 1ull);
  }

  // top-K of the biased scores among eligible experts
  int my_e = 0;
  float my_s = 0.0f;
  float ssum = 0.0f, last_c = 0.0f;
  for (int k = 0; k <= K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      const bool ok = elig[j] && !taken[j];
      if (ok && better(c[j], e, bv, bi)) { bv = c[j]; bi = e; }
    }
    wave_argmax(bv, bi);
    if (k == K) {  // the (K+1)-th best, for the near-tie flag only
      if (bi != 0x7fffffff && last_c - bv <= p.eps) tie = true;
      break;
    }
    const float sw = s_row[bi];
    ssum = (k == 0) ? sw : ssum + sw;
    if (lane == k) { my_e = bi; my_s = sw; }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + kWave * j == bi) taken[j] = true;
    last_c = bv;
  }
  if (lane < K) {
    const float g = (ssum == 0.0f) ? 1.0f / static_cast<float>(K) : my_s / ssum;
    idx_out[t * K + lane] = my_e;
    gate_out[t * K + lane] = g;
    atomicAdd(&hist[my_e], 1);
  }
  if (lane == 0 && tie) atomicAdd(ntie, 1);
  // the rows are rewritten for this wave's next token only after every lane
  // has read them
  wave_lds_sync();
}

}  // namespace
}  // namespace dsmoe
