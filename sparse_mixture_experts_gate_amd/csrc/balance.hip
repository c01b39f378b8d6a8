// Sequence-level balance loss of the router and its gradient on gfx950.
//
// The training-techniques article (mhpq.cn "DeepSeek-V3 高效训练关键技术全景
// 解析" §1.2) adds, next to the bias-based balancing, a per-sequence balance
// loss that keeps the tokens of one sequence from concentrating on a few
// experts; it gives no formula. Computed here, for each sequence of L
// consecutive tokens, with the layer's fp32 logits u and its selection:
//   s = sigmoid(u) over all E experts, S_t = sum_i s_ti, s'_ti = s_ti / S_t
//       (1/E where every fp32 score of the token is zero);
//   P_i = (1/L) sum_t s'_ti,  f_i = E / (K L) * (routed slots of expert i);
//   loss = alpha * sum_i f_i P_i;
//   du_tj = alpha / (L S_t) * (f_j - F_t) * s_tj (1 - s_tj)
//         = (alpha / L) * (g_j - G_t) * s'_tj * (1 - s_tj),
//       F_t = sum_i f_i s'_ti, g = f - 1, G_t = sum_i g_i s'_ti (the same
//       difference, since sum_i s'_ti = 1, without the cancellation of two
//       numbers near 1 at balance; f is piecewise constant: no gradient);
// then dWr = du^T x and dx = du Wr as two k-major weight-gradient GEMMs
// (backward.hip), one contracting over the tokens, one over the experts.
//
// Every sum runs in a fixed order (per wave in token order, waves and
// chunks in index order), so the results do not depend on scheduling.
#include "device_common.h"
#include "internal.h"
#include "sigmoid_ieee.h"

namespace dsmoe {
namespace {

constexpr int kChunk = kBalanceChunk;
constexpr int kTokU = 4;            // tokens per wave and step, loads issued together
constexpr int kMaxJ = 8;            // experts per lane: E <= 512
constexpr int kThreads = 256;       // 4 waves

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Partial sums of one chunk of kChunk tokens inside one sequence:
// part_p[c, e] = sum over the chunk's tokens of s'_te, part_c[c, e] = routed
// slots of expert e. One workgroup per chunk: chunk c of sequence q is
// workgroup q * cps + c (cps chunks per sequence).
__global__ __launch_bounds__(kThreads) void seqbal_partial_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx, int E, int K, int L,
    int cps, float* __restrict__ part_p, int32_t* __restrict__ part_c) {
  __shared__ float wpart[4][kMaxJ * 64];
  __shared__ int hist[kMaxJ * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk = blockIdx.x;
  const int64_t q = chunk / cps;
  const int c = static_cast<int>(chunk - q * cps);
  const int64_t t0 = q * L + static_cast<int64_t>(c) * kChunk;
  const int ntok = min(kChunk, L - c * kChunk);
  const int nj = (E + 63) / 64;
  for (int e = tid; e < E; e += kThreads) hist[e] = 0;
  float acc[kMaxJ];
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j) acc[j] = 0.0f;
  const float inv_e = 1.0f / static_cast<float>(E);
  // wave w takes tokens 4w .. 4w + 3, then 16 + 4w .., in token order; the
  // logits of its four tokens are loaded before any is used
  for (int i0 = wave * kTokU; i0 < ntok; i0 += 4 * kTokU) {
    float uv[kTokU][kMaxJ];
#pragma unroll
    for (int k = 0; k < kTokU; ++k)
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) {
        const int e = lane + 64 * j;
        uv[k][j] = (i0 + k < ntok && j < nj && e < E) ? logits[(t0 + i0 + k) * E + e] : 0.0f;
      }
#pragma unroll
    for (int k = 0; k < kTokU; ++k) {
      if (i0 + k >= ntok) break;
      float sv[kMaxJ], part = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) {
        sv[j] = (j < nj && lane + 64 * j < E) ? sigmoid_ieee(uv[k][j]) : 0.0f;
        part += sv[j];
      }
      const float S = wave_sum(part);
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) acc[j] += S > 0.0f ? sv[j] / S : inv_e;
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j)
    if (j < nj) wpart[wave][lane + 64 * j] = acc[j];
  __syncthreads();
  for (int p = tid; p < ntok * K; p += kThreads) atomicAdd(&hist[idx[t0 * K + p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    part_p[chunk * E + e] = ((wpart[0][e] + wpart[1][e]) + wpart[2][e]) + wpart[3][e];
    part_c[chunk * E + e] = hist[e];
  }
}

// One workgroup per sequence: P_i, f_i, the loss, and g_i = f_i - 1 for the
// gradient.
__global__ __launch_bounds__(kThreads) void seqbal_reduce_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c, int E, int K, int L,
    int cps, float alpha, float* __restrict__ f_out, float* __restrict__ loss) {
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.x;
  const float inv_l = 1.0f / static_cast<float>(L);
  float term = 0.0f;
  for (int e = tid; e < E; e += kThreads) {
    float p = 0.0f;
    int64_t cnt = 0;
#pragma unroll 8
    for (int c = 0; c < cps; ++c) {
      p += part_p[(q * cps + c) * E + e];
      cnt += part_c[(q * cps + c) * E + e];
    }
    const double kl = static_cast<double>(K) * L;
    const float f = static_cast<float>(static_cast<double>(cnt) * E / kl);
    // the gradient uses g = f - 1, formed from the integer counts: near
    // balance f_j - F_t cancels, g_j - G_t does not
    f_out[q * E + e] = static_cast<float>((static_cast<double>(cnt) * E - kl) / kl);
    term += f * (p * inv_l);
  }
  term = wave_sum(term);
  if ((tid & 63) == 0) red[tid >> 6] = term;
  __syncthreads();
  if (tid == 0) loss[q] = alpha * (((red[0] + red[1]) + red[2]) + red[3]);
}

// du for kChunk tokens (each wave four at a time), written as fp32 [T, E]
// (optional), bf16 [T, ldE] (columns E.. ldE - 1 zero) and bf16 transposed
// [E, ldT] through an LDS tile. Grid ceil(T / kChunk).
__global__ __launch_bounds__(kThreads) void seqbal_grad_kernel(
    const float* __restrict__ logits, const float* __restrict__ f_all, int64_t T, int E, int L,
    float alpha, float* __restrict__ dlogits, uint16_t* __restrict__ du16, int ldE,
    uint16_t* __restrict__ duT16, int64_t ldT) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kMaxJ * 64][kChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kChunk;
  const int ntok = static_cast<int>(min(static_cast<int64_t>(kChunk), T - t0));
  const int nj = (E + 63) / 64, njw = (ldE + 63) / 64;
  const float a_l = alpha / static_cast<float>(L);
  for (int i0 = wave * kTokU; i0 < kChunk; i0 += 4 * kTokU) {
    // the logits of the wave's four tokens are loaded before any is used
    float uv[kTokU][kMaxJ];
#pragma unroll
    for (int k = 0; k < kTokU; ++k)
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) {
        const int e = lane + 64 * j;
        uv[k][j] = (i0 + k < ntok && j < nj && e < E) ? logits[(t0 + i0 + k) * E + e] : 0.0f;
      }
#pragma unroll
    for (int k = 0; k < kTokU; ++k) {
    const int i = i0 + k;
    const int64_t t = t0 + i;
    if (i >= ntok) {
      // columns of tokens past T: zeros in the transposed tile
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j)
        if (j < nj && lane + 64 * j < E) tile[lane + 64 * j][i] = 0;
      continue;
    }
    const float* f = f_all + (t / L) * E;
    float s[kMaxJ], fv[kMaxJ];
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int e = lane + 64 * j;
      const bool in = j < nj && e < E;
      s[j] = in ? sigmoid_ieee(uv[k][j]) : 0.0f;
      fv[j] = in ? f[e] : 0.0f;
      part += s[j];
    }
    const float S = wave_sum(part);
    // s'_j = s_j / S (zero where S is zero: no gradient); the factor
    // alpha / (L S) is applied through s', which stays finite for tiny S.
    // fv holds g = f - 1: since sum_i s'_i = 1, f_j - F_t = g_j - G_t with
    // G_t = sum_i g_i s'_i, which keeps its precision near balance
    float sn[kMaxJ], fpart = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      sn[j] = S > 0.0f ? s[j] / S : 0.0f;
      fpart += fv[j] * sn[j];
    }
    const float F = wave_sum(fpart);
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int e = lane + 64 * j;
      const float g = a_l * (fv[j] - F) * sn[j] * (1.0f - s[j]);
      if (j < nj && e < E) {
        if (dlogits) dlogits[t * E + e] = g;
        tile[e][i] = f32_to_bf16(g);
      }
      if (j < njw && e < ldE) du16[t * ldE + e] = e < E ? f32_to_bf16(g) : 0;
    }
    }
  }
  __syncthreads();
  // rows of the transposed tile: 8 tokens (16 bytes) per store, pieces that
  // start before ldT (the padding columns of the last chunk hold zeros)
  for (int p = tid; p < E * (kChunk / 8); p += kThreads) {
    const int e = p / (kChunk / 8), g = p % (kChunk / 8);
    const int64_t col = t0 + 8 * g;
    if (col >= ldT) continue;
    *reinterpret_cast<uint4*>(duT16 + e * ldT + col) = *reinterpret_cast<const uint4*>(&tile[e][8 * g]);
  }
}

// off[g] = min(g * step, T) for g = 0 .. G: the token groups over which the
// router weight gradient is split.
__global__ void token_groups_kernel(int32_t* __restrict__ off, int G, int step, int64_t T) {
  for (int g = threadIdx.x; g <= G; g += blockDim.x)
    off[g] = static_cast<int32_t>(min(static_cast<int64_t>(g) * step, T));
}

// out[i] = ((part[i] + part[n + i]) + ...) + part[(G - 1) n + i], four per
// thread; n a multiple of 4.
__global__ __launch_bounds__(kThreads) void sum_groups_kernel(const float* __restrict__ part,
                                                               int G, int64_t n4,
                                                               float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n4) return;
  const float4* p = reinterpret_cast<const float4*>(part);
  float4 a = p[i];
  for (int g0 = 1; g0 < G; g0 += 4) {
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = g0 + j < G ? p[static_cast<int64_t>(g0 + j) * n4 + i] : a;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (g0 + j < G) {
        a.x = a.x + v[j].x;
        a.y = a.y + v[j].y;
        a.z = a.z + v[j].z;
        a.w = a.w + v[j].w;
      }
  }
  reinterpret_cast<float4*>(out)[i] = a;
}

// dst[i] = bf16(src[i]), 8 per thread; n a multiple of 8.
__global__ __launch_bounds__(kThreads) void to_bf16_kernel(const float* __restrict__ src,
                                                            int64_t n8, uint16_t* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
  reinterpret_cast<uint4*>(dst)[i] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w),
                                                pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
}

}  // namespace

hipError_t launch_seq_balance(const float* logits, const int32_t* idx, int64_t T, int E, int K,
                              int L, float alpha, float* part_p, int32_t* part_c, float* f,
                              float* loss, float* dlogits, uint16_t* du16, int ldE,
                              uint16_t* duT16, int64_t ldT, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cps = (L + kChunk - 1) / kChunk;
  const unsigned n_seq = static_cast<unsigned>(T / L);
  hipLaunchKernelGGL(seqbal_partial_kernel, dim3(static_cast<unsigned>(n_seq * cps)),
                     dim3(kThreads), 0, s, logits, idx, E, K, L, cps, part_p, part_c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seqbal_reduce_kernel, dim3(n_seq), dim3(kThreads), 0, s, part_p, part_c, E,
                     K, L, cps, alpha, f, loss);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nchunks = static_cast<unsigned>((T + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(seqbal_grad_kernel, dim3(nchunks), dim3(kThreads), 0, s, logits, f, T, E, L,
                     alpha, dlogits, du16, ldE, duT16, ldT);
  return hipGetLastError();
}

hipError_t launch_token_groups(int32_t* off, int G, int step, int64_t T, hipStream_t s) {
  hipLaunchKernelGGL(token_groups_kernel, dim3(1), dim3(64), 0, s, off, G, step, T);
  return hipGetLastError();
}

hipError_t launch_sum_groups(const float* part, int G, int64_t n, float* out, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(sum_groups_kernel, dim3(static_cast<unsigned>((n4 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, part, G, n4, out);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, int64_t n, uint16_t* dst, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(static_cast<unsigned>((n8 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, src, n8, dst);
  return hipGetLastError();
}

}  // namespace dsmoe
