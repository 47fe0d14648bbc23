// Fresh partial attention state, bf16 inputs, MFMA with fp32 accumulation (gfx950).
//
// Computes, for one query partition against one K/V partition (the "attention
// state" of the DiTango page, State-Centric Parallel Runtime > State
// Composition):
//     S = scale * Q K^T,   LSE = ln sum_j exp(S_ij),   O = exp(S - LSE) V
// as a single pass over the key tiles with a running (online) maximum.
//
// Mapping onto CDNA4
// ------------------
// * A workgroup owns BM = 128 queries of one (batch, head) and one fresh
//   partition (grid.z selects the job of a grouped launch); each of its four
//   waves owns 32 queries.
// * Scores are produced transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16: the A operand is a 32-key x 16-dim slice of the
//   K tile (LDS), the B operand the wave's Q^T slice, held in registers for
//   the whole kernel.  In the 32x32 accumulator every lane then owns ONE query
//   (column) and 16 of the 32 keys; its partner lane (lane ^ 32) owns the
//   other 16.  Row max and row sum need no more than one cross-lane exchange.
// * The probabilities feed O^T += V^T P^T directly from registers: for the
//   B operand a lane must supply 8 keys of its own query, and the 8
//   accumulator entries of one half of the S^T block are exactly that (keys
//   {0-3, 8-11} in the low half-wave, {4-7, 12-15} in the high one).  V^T is
//   laid out in LDS with the same key permutation inside every group of 16
//   keys, so the A operand is one 16-byte LDS read per lane.
// * The output accumulator O^T again gives each lane one query, so the
//   online-softmax rescale and the final 1/l are per-lane scalars.
// * Rescaling is lazy: the running max only moves (and O, l are rescaled) when
//   a tile's max exceeds it by more than 2^8 in the exp2 domain; otherwise the
//   stale max is kept, which is exact because numerator and denominator use
//   the same reference.
// * K and V tiles are fetched into registers one tile ahead (coalesced
//   16-byte loads) and written to double-buffered LDS: K row-major with a
//   16-byte row pad, V transposed with a 16-byte row pad.  One barrier per tile.
// * Ragged tails: query rows past Nq load a clamped row and are not stored;
//   key rows past nk load a clamped row and their scores are set to -inf.

#include "dita_kernels.h"

#include <cmath>

namespace dita {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the running max

template <int D>
struct Tile {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BM = kWaves * 32;           // queries per workgroup
  static constexpr int BN = 8192 / D;              // keys per tile: 64 (D=128), 128 (D=64)
  static constexpr int KS = D + 8;                 // K row stride in LDS (elements)
  static constexpr int VS = BN + 8;                // V^T row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = BN * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int V_GROUPS = BN / 4;                 // 4-key groups per tile
  static_assert(V_GROUPS * (D / 8) == kThreads, "one 4x8 V block per thread");
  static_assert(K_CHUNKS * kThreads * 8 == BN * D, "K tile split");
};

__device__ inline u32x4 load16(const __bf16* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Position, inside the V^T row of a tile, of key 4*g (the 4-key group g).
// Inside every 16-key group, key 8a + 4h + r lives at 8h + 4a + r.
__device__ inline int vt_pos(int g) { return 16 * (g >> 2) + 8 * (g & 1) + 4 * ((g >> 1) & 1); }

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(const __bf16* __restrict__ q,
                                                            AttnJobs jobs, int64_t Nq,
                                                            float scale_log2) {
  using T = Tile<D>;
  constexpr int NB = T::BN / 32;   // 32-key blocks per tile
  constexpr int NKK = D / 16;      // MFMA k-steps over the head dim
  constexpr int ND = D / 32;       // 32-wide blocks of the head dim

  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * T::BUF_ELEMS];

  const AttnJob& job = jobs.job[blockIdx.z];
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t nk = job.nk;

  const __bf16* __restrict__ kp = static_cast<const __bf16*>(job.k) + bh * nk * D;
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(job.v) + bh * nk * D;
  const __bf16* __restrict__ qp = q + bh * Nq * D;

  // Q^T operand: lane holds Q[row][kk*16 + 8*hh .. +7] for every k-step kk.
  const int64_t qrow = int64_t(blockIdx.x) * T::BM + wave * 32 + m32;
  const int64_t qrow_c = qrow < Nq ? qrow : Nq - 1;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = as_bf16x8(load16(qp + qrow_c * D + kk * 16 + 8 * hh));

  f32x16 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = zero16();
  float m_run = -INFINITY;  // running max, exp2 domain
  float l_run = 0.0f;       // this lane's partial denominator (its 16 keys per block)

  const int ntiles = int((nk + T::BN - 1) / T::BN);

  // Per-thread global->register staging of one tile.
  u32x4 kreg[T::K_CHUNKS];
  u32x4 vreg[4];
  const int vg = tid % T::V_GROUPS;  // 4-key group
  const int vc = tid / T::V_GROUPS;  // 8-wide head-dim chunk

  auto fetch = [&](int t) {
    const int64_t kbase = int64_t(t) * T::BN;
#pragma unroll
    for (int i = 0; i < T::K_CHUNKS; ++i) {
      const int id = tid + i * T::kThreads;
      const int row = id / (D / 8);
      const int col = id % (D / 8);
      int64_t r = kbase + row;
      r = r < nk ? r : nk - 1;
      kreg[i] = load16(kp + r * D + col * 8);
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      int64_t r = kbase + 4 * vg + r4;
      r = r < nk ? r : nk - 1;
      vreg[r4] = load16(vp + r * D + vc * 8);
    }
  };

  auto stash = [&](__bf16* ks, __bf16* vs) {
#pragma unroll
    for (int i = 0; i < T::K_CHUNKS; ++i) {
      const int id = tid + i * T::kThreads;
      const int row = id / (D / 8);
      const int col = id % (D / 8);
      *reinterpret_cast<u32x4*>(ks + row * T::KS + col * 8) = kreg[i];
    }
    const int pos = vt_pos(vg);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // head-dim 8*vc + 2w (low halves) and 8*vc + 2w + 1 (high halves) of the 4 keys
      u32x2 lo, hi;
      lo[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
      lo[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
      hi[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
      hi[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
      *reinterpret_cast<u32x2*>(vs + (8 * vc + 2 * w) * T::VS + pos) = lo;
      *reinterpret_cast<u32x2*>(vs + (8 * vc + 2 * w + 1) * T::VS + pos) = hi;
    }
  };

  fetch(0);
  for (int t = 0; t < ntiles; ++t) {
    __bf16* ks = smem + (t & 1) * T::BUF_ELEMS;
    __bf16* vs = ks + T::K_ELEMS;
    stash(ks, vs);
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);

    // S^T = K Q^T for the tile: NB blocks of 32 keys x 32 queries.
    f32x16 s[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s[b] = zero16();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const u32x4*>(ks + (b * 32 + m32) * T::KS + kk * 16 + 8 * hh));
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[b], 0, 0, 0);
      }
    }

    // Keys past the partition end score -inf.
    if (int64_t(t + 1) * T::BN > nk) {
      const int64_t kb0 = int64_t(t) * T::BN;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = kb0 + b * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= nk) s[b][i] = -INFINITY;
        }
    }

    // Row max of raw scores (scale > 0 commutes with max), then the pair exchange.
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = mx * scale_log2;
    const float m_new = fmaxf(m_run, m_tile);
    if (__any(m_new > m_run + kRescaleSlack)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      m_run = m_new;
    }

    // P = exp2(S * scale*log2e - m): fp32 for the denominator (so LSE keeps fp32
    // accuracy), rounded to bf16 for the P V product.
    bf16x8 pb[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 v;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * h2 + j], scale_log2, -m_run));
          part += e;
          v[j] = (__bf16)e;
        }
        l_run += part;
        pb[b][h2] = v;
      }

    // O^T += V^T P^T.
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
              vs + (d * 32 + m32) * T::VS + b * 32 + h2 * 16 + 8 * hh));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[b][h2], oacc[d], 0, 0, 0);
        }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow >= Nq) return;
  const float inv = 1.0f / l_tot;
  __bf16* __restrict__ op = static_cast<__bf16*>(job.o) + bh * Nq * D + qrow * D;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(oacc[d][4 * j + r] * inv);
      *reinterpret_cast<bf16x4*>(op + d * 32 + 8 * j + 4 * hh) = v;
    }
  if (hh == 0) job.lse[bh * Nq + qrow] = (m_run + __builtin_log2f(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_attn_bf16(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                            hipStream_t stream) {
  const float sl2 = pr.scale * kLog2e;
  if (pr.D == 128) {
    using T = Tile<128>;
    dim3 grid(unsigned((pr.Nq + T::BM - 1) / T::BM), unsigned(pr.BH), unsigned(n_jobs));
    attn_fwd_bf16_kernel<128><<<grid, T::kThreads, 0, stream>>>(static_cast<const __bf16*>(q), jobs,
                                                                pr.Nq, sl2);
  } else {
    using T = Tile<64>;
    dim3 grid(unsigned((pr.Nq + T::BM - 1) / T::BM), unsigned(pr.BH), unsigned(n_jobs));
    attn_fwd_bf16_kernel<64><<<grid, T::kThreads, 0, stream>>>(static_cast<const __bf16*>(q), jobs,
                                                               pr.Nq, sl2);
  }
  return hipGetLastError();
}

}  // namespace dita
