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
    int32_t* __restrict__ tmap1, int32_t* __restrict__ tmap2, PlanParams p) {
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
    // tile -> group maps: every thread takes tiles i, i + 1024, ... and finds
    // the group g with s[g-1] <= i < s[g] (inclusive prefix) by binary search
    auto fill = [&](const int* s, int32_t* tmap) {
      const int total = s[ng - 1];
      for (int i = tid; i < total; i += kPlanThreads) {
        int lo = 0, hi = ng - 1;  // smallest g with s[g] > i
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s[mid] > i) hi = mid; else lo = mid + 1;
        }
        tmap[i] = lo;
      }
    };
    if (tmap1) fill(s1, tmap1);
    if (tmap2) fill(s2, tmap2);
  }
}

// One workgroup per expert: scans every (t, k) pair in token order and gives
// the matches consecutive positions, so the order inside an expert is the
// ascending token order without depending on atomics.
__global__ __launch_bounds__(256) void permute_kernel(const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ offsets,
                                                     int64_t T, int K, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
  __shared__ int wsum[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = offsets[e];
  if (offsets[e + 1] == base) return;
  int running = 0;
  for (int64_t t0 = 0; t0 < T; t0 += 256) {
    const int64_t t = t0 + tid;
    int slot = -1;
    if (t < T) {
      const int32_t* row = idx + t * K;
      for (int k = 0; k < K; ++k)
        if (row[k] == e) slot = k;
    }
    const bool hit = slot >= 0;
    const uint64_t bal = __ballot(hit);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pre += q < w ? wsum[q] : 0;
      tot += wsum[q];
    }
    if (hit) {
      const int pos = base + running + pre + rank;
      if (pos < T * K) {  // guards counts that disagree with topk_idx
        perm[pos] = static_cast<int32_t>(t);
        inv[t * K + slot] = pos;
      }
    }
    running += tot;
    __syncthreads();
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
                       int32_t* tiles1, int32_t* tiles2, int32_t* tmap1, int32_t* tmap2,
                       const PlanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, counts, offsets_in,
                     offsets_out, tiles1, tiles2, tmap1, tmap2, p);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const int32_t* offsets, int64_t T, int K, int E,
                          int32_t* perm, int32_t* inv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3(E), dim3(256), 0, s, idx, offsets, T, K, perm, inv);
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
