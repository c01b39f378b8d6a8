// fp32 expert FFNs for fp32 activations and weights: one thread per output
// element, fp32 FMA accumulation. Used for small fp32 layers, where exact
// single-precision arithmetic matters more than speed.
#include "device_common.h"
#include "internal.h"

namespace dsmoe {

namespace {

// Routed expert owning row r of the permuted layout (empty experts skipped).
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // invariant: offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn1_f32_kernel(FfnArgs a) {
  const int64_t rows = a.TK + (a.Is > 0 ? a.T : 0);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * a.ldh) return;
  const int64_t row = i / a.ldh;
  const int col = static_cast<int>(i % a.ldh);
  const float* src;
  const float* W;
  int Ig;
  if (row < a.TK) {
    const int g = expert_of_row(a.offsets, a.E, static_cast<int>(row));
    Ig = a.I;
    if (a.perm) {
      const int tok = a.perm[row];
      if (tok < 0 || tok >= a.T) return;
      src = static_cast<const float*>(a.x) + static_cast<int64_t>(tok) * a.d;
    } else {
      src = static_cast<const float*>(a.xperm) + row * a.d;
    }
    W = static_cast<const float*>(a.w13) + static_cast<int64_t>(g) * 2 * a.I * a.d;
  } else {
    Ig = a.Is;
    src = static_cast<const float*>(a.x) + (row - a.TK) * a.d;
    W = static_cast<const float*>(a.ws13);
  }
  if (col >= Ig) return;
  const float* wg = W + static_cast<int64_t>(col) * a.d;
  const float* wu = W + static_cast<int64_t>(Ig + col) * a.d;
  float g = 0.0f, u = 0.0f;
  for (int k = 0; k < a.d; ++k) {
    g = __builtin_fmaf(src[k], wg[k], g);
    u = __builtin_fmaf(src[k], wu[k], u);
  }
  static_cast<float*>(a.H)[row * a.ldh + col] = silu_f32(g) * u;
}

__global__ __launch_bounds__(256) void ffn2_f32_kernel(FfnArgs a) {
  const int64_t rows = a.TK + (a.Is > 0 ? a.T : 0);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * a.d) return;
  const int64_t row = i / a.d;
  const int n = static_cast<int>(i % a.d);
  const float* h = static_cast<const float*>(a.H) + row * a.ldh;
  const float* W;
  int Ig;
  float* out;
  if (row < a.TK) {
    const int g = expert_of_row(a.offsets, a.E, static_cast<int>(row));
    Ig = a.I;
    W = static_cast<const float*>(a.w2) + static_cast<int64_t>(g) * a.d * a.I;
    out = static_cast<float*>(a.yperm) + row * a.d + n;
  } else {
    Ig = a.Is;
    W = static_cast<const float*>(a.ws2);
    out = static_cast<float*>(a.yshared) + (row - a.TK) * a.d + n;
  }
  const float* w = W + static_cast<int64_t>(n) * Ig;
  float acc = 0.0f;
  for (int k = 0; k < Ig; ++k) acc = __builtin_fmaf(h[k], w[k], acc);
  *out = acc;
}

}  // namespace

hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s, hipEvent_t mid) {
  const int64_t rows = a.TK + (a.Is > 0 ? a.T : 0);
  if (rows == 0) return hipSuccess;
  const int64_t n1 = rows * a.ldh, n2 = rows * a.d;
  hipLaunchKernelGGL(ffn1_f32_kernel, dim3(static_cast<unsigned>((n1 + 255) / 256)), dim3(256), 0,
                     s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(ffn2_f32_kernel, dim3(static_cast<unsigned>((n2 + 255) / 256)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace dsmoe
