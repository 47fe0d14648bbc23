// Statistics the error-guided planner reads (the DiTango page, Methodology >
// 1. Anchor-Guided Selection Planner: "Error Modeling" needs each partition's
// importance, "Online Prediction" the change of the always-computed local
// state).
//
// contrib_kernel: w_p = mean over rows of exp(LSE_p - LSE), the share of
//   partition p in the merged softmax.  One workgroup per partition reads two
//   fp32 LSE arrays (8 bytes per row); fp64 accumulation, fixed reduction
//   order (deterministic).  Run at anchor steps only: at the 75,600-token
//   shape 16 x 189,000 rows, ~12 MB.
// change_kernel: sums of (a - b)^2 and b^2 over two output states, fp64 per
//   lane, a fixed-order workgroup reduction, one partial pair per workgroup
//   into a scratch buffer; optionally copies a over b (state and LSE) in the
//   same pass.  HBM-bound: reads 2 states, writes one when rolling.
// change_finish_kernel: one workgroup adds the partials in a fixed order and
//   forms the ratio sqrt(sum (a-b)^2 / sum b^2).  The grid depends only on the
//   state's size, so the result is the same bit for bit on every run.

#include "dita_kernels.h"

#include <cmath>

namespace dita {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 1024;
constexpr int kChangeThreads = 256;
constexpr int kChangeItems = kChangeThreads * 8;  // 16-byte chunks per workgroup before the cap

__device__ double block_sum(double v, double* red) {
  // wave reduction, then one value per wave through LDS
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const int nw = blockDim.x >> 6;
  double s = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < nw; ++w) s += red[w];
  return s;  // valid in thread 0
}

__global__ __launch_bounds__(kThreads) void contrib_kernel(LseList src, const float* __restrict__ lse,
                                                           int64_t rows, double* __restrict__ w) {
  __shared__ double red[kThreads / 64];
  const int p = blockIdx.x;
  const float* lp = src.lse[p];
  double acc = 0.0;
  for (int64_t r = threadIdx.x; r < rows; r += kThreads) {
    const float l = lse[r], a = lp[r];
    if (l != -INFINITY && a != -INFINITY) acc += exp(double(a) - double(l));
  }
  const double s = block_sum(acc, red);
  if (threadIdx.x == 0) w[p] = s / double(rows);
}

template <typename T>
__device__ void widen(u32x4 r, double* x);
template <>
__device__ void widen<float>(u32x4 r, double* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = r[i];
    x[i] = double(__builtin_bit_cast(float, u));
  }
}
template <>
__device__ void widen<__bf16>(u32x4 r, double* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = r[i];
    x[2 * i] = double(__builtin_bit_cast(float, u << 16));
    x[2 * i + 1] = double(__builtin_bit_cast(float, u & 0xffff0000u));
  }
}

template <typename T>
__global__ __launch_bounds__(kChangeThreads) void change_kernel(const u32x4* __restrict__ a,
                                                                u32x4* __restrict__ b, int64_t n16,
                                                                const float* __restrict__ la,
                                                                float* __restrict__ lb, int64_t nl,
                                                                int roll, double* __restrict__ part) {
  __shared__ double red[kChangeThreads / 64];
  constexpr int N = 16 / sizeof(T);
  const int64_t stride = int64_t(gridDim.x) * kChangeThreads;
  double d2 = 0.0, b2 = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * kChangeThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 ra = __builtin_nontemporal_load(a + i);
    const u32x4 rb = b[i];
    double xa[N], xb[N];
    widen<T>(ra, xa);
    widen<T>(rb, xb);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const double d = xa[j] - xb[j];
      d2 = fma(d, d, d2);
      b2 = fma(xb[j], xb[j], b2);
    }
    if (roll) b[i] = ra;
  }
  if (roll)
    for (int64_t i = int64_t(blockIdx.x) * kChangeThreads + threadIdx.x; i < nl; i += stride)
      lb[i] = la[i];
  const double s_d = block_sum(d2, red);
  __syncthreads();
  const double s_b = block_sum(b2, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = s_d;
    part[2 * blockIdx.x + 1] = s_b;
  }
}

// Thread t adds the partials of workgroups t, t + 256, ... in order; the
// workgroup sum then runs in the fixed order of block_sum.
__global__ __launch_bounds__(kChangeThreads) void change_finish_kernel(const double* __restrict__ part,
                                                                       int groups,
                                                                       double* __restrict__ out) {
  __shared__ double red[kChangeThreads / 64];
  double d = 0.0, b = 0.0;
  for (int g = threadIdx.x; g < groups; g += kChangeThreads) {
    d += part[2 * g];
    b += part[2 * g + 1];
  }
  const double num = block_sum(d, red);
  __syncthreads();
  const double den = block_sum(b, red);
  if (threadIdx.x == 0) {
    out[0] = num;
    out[1] = den;
    out[2] = den > 0.0 ? sqrt(num / den) : (num > 0.0 ? INFINITY : 0.0);
  }
}

}  // namespace

hipError_t launch_contrib(int P, const LseList& src, const float* lse, int64_t rows, double* w,
                          hipStream_t stream) {
  contrib_kernel<<<dim3(unsigned(P)), kThreads, 0, stream>>>(src, lse, rows, w);
  return hipGetLastError();
}

int change_groups(size_t o_bytes) {
  const int64_t n16 = int64_t(o_bytes / 16);
  int64_t g = (n16 + kChangeItems - 1) / kChangeItems;
  if (g > kChangeMaxGroups) g = kChangeMaxGroups;
  return g < 1 ? 1 : int(g);
}

hipError_t launch_change(int dtype, const void* o_new, void* o_prev, size_t o_bytes,
                         const float* lse_new, float* lse_prev, size_t lse_bytes, int roll,
                         double* partials, double* out, hipStream_t stream) {
  const int64_t n16 = int64_t(o_bytes / 16), nl = int64_t(lse_bytes / 4);
  const int groups = change_groups(o_bytes);
  const u32x4* a = static_cast<const u32x4*>(o_new);
  u32x4* b = static_cast<u32x4*>(o_prev);
  if (dtype == 1)
    change_kernel<__bf16><<<dim3(unsigned(groups)), kChangeThreads, 0, stream>>>(
        a, b, n16, lse_new, lse_prev, nl, roll, partials);
  else
    change_kernel<float><<<dim3(unsigned(groups)), kChangeThreads, 0, stream>>>(
        a, b, n16, lse_new, lse_prev, nl, roll, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  change_finish_kernel<<<1, kChangeThreads, 0, stream>>>(partials, groups, out);
  return hipGetLastError();
}

}  // namespace dita
