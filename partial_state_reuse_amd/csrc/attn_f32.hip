// Fresh partial attention state in fp32 throughout (no reduced-precision step).
//
// Same contract as the bf16 kernel (the attention state of the DiTango page,
// State-Centric Parallel Runtime > State Composition):
//     S = scale * Q K^T,   LSE = ln sum_j exp(S_ij),   O = exp(S - LSE) V
// One lane owns one query row; K and V tiles of 32 keys are staged through
// LDS and read as broadcasts.  Online softmax with a running max; every
// product, exponential and sum is fp32.  This path serves fp32 inputs, whose
// sizes here are small; it is not tuned for throughput.

#include "dita_kernels.h"

#include <cmath>

namespace dita {
namespace {

constexpr int kRows = 64;   // queries per workgroup (one wave)
constexpr int kTileK = 32;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void attn_fwd_f32_kernel(const float* __restrict__ q,
                                                             AttnJobs jobs, int64_t Nq,
                                                             float scale) {
  __shared__ float ks[kTileK][D];
  __shared__ float vs[kTileK][D];

  const AttnJob& job = jobs.job[blockIdx.z];
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t nk = job.nk;
  const float* __restrict__ kp = static_cast<const float*>(job.k) + bh * nk * D;
  const float* __restrict__ vp = static_cast<const float*>(job.v) + bh * nk * D;
  const int64_t row = int64_t(blockIdx.x) * kRows + tid;
  const int64_t rc = row < Nq ? row : Nq - 1;

  float qr[D];
  const float* qrow = q + (bh * Nq + rc) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = qrow[d];
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  for (int64_t k0 = 0; k0 < nk; k0 += kTileK) {
    const int nt = int(nk - k0 < kTileK ? nk - k0 : kTileK);
    for (int i = tid; i < kTileK * D; i += kRows) {
      const int r = i / D, c = i % D;
      ks[r][c] = r < nt ? kp[(k0 + r) * D + c] : 0.0f;
      vs[r][c] = r < nt ? vp[(k0 + r) * D + c] : 0.0f;
    }
    __syncthreads();
    float s[kTileK];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTileK; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qr[d], ks[j][d], acc);
      s[j] = j < nt ? acc * scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    const float alpha = expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kTileK; ++j) {
      const float p = expf(s[j] - mn);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vs[j][d], o[d]);
    }
    m = mn;
    __syncthreads();
  }
  if (row >= Nq) return;
  const float inv = 1.0f / l;
  float* orow = static_cast<float*>(job.o) + (bh * Nq + row) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
  job.lse[bh * Nq + row] = m + logf(l);
}

}  // namespace

hipError_t launch_attn_f32(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                           hipStream_t stream) {
  dim3 grid(unsigned((pr.Nq + kRows - 1) / kRows), unsigned(pr.BH), unsigned(n_jobs));
  if (pr.D == 128)
    attn_fwd_f32_kernel<128><<<grid, kRows, 0, stream>>>(static_cast<const float*>(q), jobs, pr.Nq,
                                                         pr.scale);
  else
    attn_fwd_f32_kernel<64><<<grid, kRows, 0, stream>>>(static_cast<const float*>(q), jobs, pr.Nq,
                                                        pr.scale);
  return hipGetLastError();
}

}  // namespace dita
