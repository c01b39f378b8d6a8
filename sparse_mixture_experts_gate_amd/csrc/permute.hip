// Per-expert token segments: exclusive scan of the per-expert counts, a
// stable counting sort of the (token, slot) pairs by expert, and the tile
// tables of the persistent grouped GEMMs. Segments are sized to the routed
// data, the one-GPU counterpart of all-to-all buffers opened for the data
// actually sent (mhpq.cn "DeepSeek-V3 高效训练关键技术全景解析" §3.1).
#include "device_common.h"
#include "internal.h"

namespace dsmoe {

namespace {

constexpr int kPlanThreads = 1024;

// Inclusive scan of v[0..n) in LDS (n <= kPlanThreads), all threads call it.
__device__ void block_inclusive_scan(int* v, int n, int* tmp) {
  const int tid = threadIdx.x;
  for (int off = 1; off < n; off <<= 1) {
    int add = 0;
    if (tid < n && tid >= off) add = v[tid - off];
    __syncthreads();
    if (tid < n) v[tid] += add;
    __syncthreads();
  }
  (void)tmp;
}

// Single workgroup. Group g < E is routed expert g (rows = its count); group E
// is the shared expert (rows = T, or none when Is == 0).
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets_in,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ tiles1, int32_t* __restrict__ tiles2,
    PlanParams p) {
  __shared__ int rows[kPlanThreads];
  __shared__ int s1[kPlanThreads];
  __shared__ int s2[kPlanThreads];
  const int tid = threadIdx.x;
  const int E = p.E;
  const int ng = E + 1;
  if (tid < E) rows[tid] = counts ? counts[tid] : offsets_in[tid + 1] - offsets_in[tid];
  if (tid == E) rows[tid] = p.Is > 0 ? static_cast<int>(p.T) : 0;
  if (tid > E) rows[tid] = 0;
  __syncthreads();
  // tiles per group for both GEMMs
  if (tid < ng) {
    const int r = rows[tid];
    const int ig = tid == E ? p.Is : p.I;
    const int nt1 = ig > 0 ? (ig + p.bnh1 - 1) / p.bnh1 : 0;
    const int nt2 = (p.d + p.bn2 - 1) / p.bn2;
    s1[tid] = ((r + p.bm1 - 1) / p.bm1) * nt1;
    s2[tid] = ((r + p.bm2 - 1) / p.bm2) * nt2;
  } else {
    s1[tid] = 0;
    s2[tid] = 0;
  }
  __syncthreads();
  if (offsets_out) {
    // offsets: exclusive scan of the routed counts (reuse rows[] in place)
    block_inclusive_scan(rows, E, nullptr);
    if (tid == 0) offsets_out[0] = 0;
    if (tid < E) offsets_out[tid + 1] = rows[tid];
  }
  if (tiles1 || tiles2) {
    block_inclusive_scan(s1, ng, nullptr);
    block_inclusive_scan(s2, ng, nullptr);
    if (tid == 0) {
      if (tiles1) tiles1[0] = 0;
      if (tiles2) tiles2[0] = 0;
    }
    if (tid < ng) {
      if (tiles1) tiles1[tid + 1] = s1[tid];
      if (tiles2) tiles2[tid + 1] = s2[tid];
    }
  }
}

// One workgroup per expert: scans the flat selections idx[t * K + k] in
// order and gives the matches consecutive positions, so the order inside an
// expert is the ascending token order (a token selects an expert at most
// once, so flat order is token order) without depending on atomics. Each
// thread owns kPermEnt consecutive flat entries per pass, read with 16-byte
// buffer loads (coalesced across the wave); the next pass's loads are issued
// before the current pass is placed; a workgroup-wide exclusive scan of the
// per-thread match counts places the matches.
constexpr int kPermThreads = 1024;
constexpr int kPermEnt = 16;  // four 16-byte loads
constexpr int64_t kPermPass = static_cast<int64_t>(kPermThreads) * kPermEnt;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ offsets,
                                                              int64_t T, int K,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv) {
  __shared__ int wsum[kPermThreads / 64];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = offsets[e];
  if (offsets[e + 1] == base) return;
  const int64_t TK = T * K;
  // flat entries past TK read as zeros (range-checked) and are masked below
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(idx), static_cast<short>(0),
                                        static_cast<int>(TK * 4), 0x00020000);
  auto load = [&](int64_t pass, uint4 (&v)[kPermEnt / 4]) {
    const int64_t f0 = pass * kPermPass + static_cast<int64_t>(tid) * kPermEnt;
#pragma unroll
    for (int q = 0; q < kPermEnt / 4; ++q) {
      const int64_t f = f0 + 4 * q;
      v[q] = f < TK ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    r, static_cast<uint32_t>(f * 4), 0, 0))
                    : make_uint4(0, 0, 0, 0);
    }
  };
  const int64_t npass = (TK + kPermPass - 1) / kPermPass;
  uint4 cur[kPermEnt / 4], nxt[kPermEnt / 4];
  load(0, cur);
  int running = 0;
  for (int64_t pass = 0; pass < npass; ++pass) {
    if (pass + 1 < npass) load(pass + 1, nxt);
    const int64_t f0 = pass * kPermPass + static_cast<int64_t>(tid) * kPermEnt;
    uint32_t match = 0;  // bit j: entry f0 + j selects expert e
#pragma unroll
    for (int q = 0; q < kPermEnt / 4; ++q) {
      const int32_t v4[4] = {static_cast<int32_t>(cur[q].x), static_cast<int32_t>(cur[q].y),
                             static_cast<int32_t>(cur[q].z), static_cast<int32_t>(cur[q].w)};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v4[j] == e && f0 + 4 * q + j < TK) match |= 1u << (4 * q + j);
    }
    const int mine = __builtin_popcount(match);
    // inclusive scan of `mine` inside the wave, then across the waves
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < kPermThreads / 64; ++q) {
      pre += q < w ? wsum[q] : 0;
      tot += wsum[q];
    }
    int pos = base + running + pre + incl - mine;
    while (match) {
      const int j = __builtin_ctz(match);
      match &= match - 1;
      const int64_t f = f0 + j;
      if (pos < TK) {  // guards counts that disagree with topk_idx
        perm[pos] = static_cast<int32_t>(f / K);
        inv[f] = pos;
      }
      ++pos;
    }
    running += tot;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPermEnt / 4; ++q) cur[q] = nxt[q];
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ src,
                                                          const int32_t* __restrict__ perm,
                                                          int64_t n_src, int64_t row_bytes,
                                                          uint8_t* __restrict__ dst) {
  const int64_t i = blockIdx.x;
  const int64_t r = perm[i];
  uint4* d = reinterpret_cast<uint4*>(dst + i * row_bytes);
  const int64_t n = row_bytes / 16;
  if (r < 0 || r >= n_src) {  // out-of-range ids gather zeros
    for (int64_t c = threadIdx.x; c < n; c += blockDim.x) d[c] = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint4* s = reinterpret_cast<const uint4*>(src + r * row_bytes);
  for (int64_t c = threadIdx.x; c < n; c += blockDim.x) d[c] = s[c];
}

}  // namespace

hipError_t launch_plan(const int32_t* counts, const int32_t* offsets_in, int32_t* offsets_out,
                       int32_t* tiles1, int32_t* tiles2, const PlanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, counts, offsets_in,
                     offsets_out, tiles1, tiles2, p);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const int32_t* offsets, int64_t T, int K, int E,
                          int32_t* perm, int32_t* inv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3(E), dim3(kPermThreads), 0, s, idx, offsets, T, K, perm,
                     inv);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, int64_t n_src, const int32_t* perm, int64_t n,
                              int64_t row_bytes, void* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(n)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), perm, n_src, row_bytes,
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace dsmoe
