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
//   partition of a grouped launch; each of its four waves owns 32 queries.
//   Workgroup ids are remapped so that all query tiles of one (head,
//   partition) run on the same XCD and share its L2 copy of K and V.
// * K and V tiles (BN keys x D) travel HBM -> LDS with direct-to-LDS loads
//   (global_load_lds_dwordx4): no staging registers.  Both stay row-major in
//   LDS with the 16-byte chunks of each row XOR-swizzled (chunk c of row r at
//   c ^ swz(r)) so that the K reads and the transposed V reads below are free
//   of bank conflicts.  Two stages; one barrier per tile.
// * Scores are produced transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16: the A operand is a 32-key x 16-dim slice of the
//   K tile, the B operand the wave's Q^T slice, held in registers for the
//   whole kernel.  In the 32x32 accumulator every lane owns ONE query and 16
//   of the 32 keys; its partner lane (lane ^ 32) owns the other 16.
// * The probabilities feed O^T += V^T P^T directly from registers: for the
//   B operand a lane supplies 8 keys of its own query, and the 8 accumulator
//   entries of one half of an S^T block are exactly that (keys {0-3, 8-11}
//   in the low half-wave, {4-7, 12-15} in the high one).  The matching A
//   operand (8 keys x one head-dim column of V) comes from two LDS transpose
//   reads (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element
//   i%4 of the rows addressed by lanes i/4 + {0,4,8,12}, so pointing lane x
//   at key (x/4) and head-dim offset 4*(x%4) hands every lane 4 keys of its
//   own column.
// * The output accumulator O^T again gives each lane one query, so the
//   online-softmax rescale and the final 1/l are per-lane scalars.  Rescaling
//   is lazy: the running max only moves (and O, l are rescaled) when a
//   tile's max exceeds it by more than 2^8 in the exp2 domain.
// * The denominator sums the fp32 probabilities (LSE keeps fp32 accuracy);
//   the P V product uses them rounded to bf16.
// * Ragged tails: query rows past Nq load a clamped row and are not stored;
//   key rows past nk load a clamped row and their scores are set to -inf.

#include "dita_kernels.h"

#include <cmath>

namespace dita {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the running max
constexpr int kXcds = 8;

template <int D>
struct Tile {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BM = kWaves * 32;             // queries per workgroup
  static constexpr int BN = 8192 / D;                // keys per tile: 64 (D=128), 128 (D=64)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // 16 KiB
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES; // K then V
  static constexpr int NSTAGE = 2;
  static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread per tensor
  static_assert(LOADS * kThreads == BN * CPR, "tile split");
};

// Chunk swizzle of row r.  D=128 (16 chunks per row): the 16 rows read together
// by K fragments hit 16 distinct chunk slots, and the 4 consecutive rows x 4
// chunks read together by V transpose fragments hit 16 distinct slots.  D=64 (8
// chunks, two rows per 64 banks): the same two properties with row parity.
template <int D>
__device__ inline int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ inline u32x4 load16(const __bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Bijection of [0, n) that gives each XCD (workgroups are dispatched to XCDs
// round-robin) one contiguous range of logical tiles.
__device__ inline int64_t xcd_remap(int64_t pid, int64_t n) {
  const int64_t per = (n + kXcds - 1) / kXcds;
  const int64_t tall = n % kXcds == 0 ? kXcds : n % kXcds;
  const int64_t xcd = pid % kXcds, local = pid / kXcds;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const __bf16* __restrict__ q,
                                                               AttnJobs jobs, int64_t Nq, int BH,
                                                               int QT, float scale_log2) {
  using T = Tile<D>;
  constexpr int NB = T::BN / 32;   // 32-key blocks per tile
  constexpr int NKK = D / 16;      // MFMA k-steps over the head dim
  constexpr int ND = D / 32;       // 32-wide blocks of the head dim

  __shared__ __attribute__((aligned(1024))) char smem[T::NSTAGE * T::STAGE_BYTES];

  const int64_t n_tiles = int64_t(gridDim.x);
  const int64_t lin = xcd_remap(blockIdx.x, n_tiles);
  const int qt = int(lin % QT);
  const int64_t rest = lin / QT;
  const int64_t bh = rest % BH;
  const int jid = int(rest / BH);

  const AttnJob& job = jobs.job[jid];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t nk = job.nk;

  const __bf16* __restrict__ kp = static_cast<const __bf16*>(job.k) + bh * nk * D;
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(job.v) + bh * nk * D;
  const __bf16* __restrict__ qp = q + bh * Nq * D;

  // Q^T operand: lane holds Q[row][kk*16 + 8*hh .. +7] for every k-step kk.
  const int64_t qrow = int64_t(qt) * T::BM + wave * 32 + m32;
  const int64_t qrow_c = qrow < Nq ? qrow : Nq - 1;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = as_bf16x8(load16(qp + qrow_c * D + kk * 16 + 8 * hh));

  f32x16 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = zero16();
  float m_run = -INFINITY;  // running max, exp2 domain
  float l_run = 0.0f;       // this lane's partial denominator

  const int ntiles = int((nk + T::BN - 1) / T::BN);

  // Direct-to-LDS fetch of tile t into stage st: LDS slot s (16 bytes) holds
  // chunk (s % CPR) ^ swz(row) of row s / CPR.  The LDS destination of a wave's
  // load is lane-linear; the global source is chosen to match.
  auto fetch = [&](int t, int st) {
    const int64_t kbase = int64_t(t) * T::BN;
    char* kst = smem + st * T::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int s = tid + i * T::kThreads;
      const int row = s / T::CPR;
      const int c = (s % T::CPR) ^ swz<D>(row);
      int64_t r = kbase + row;
      r = r < nk ? r : nk - 1;
      const int64_t goff = r * D + c * 8;
      char* dst = kst + (wave * 64 + i * T::kThreads) * 16;
      __builtin_amdgcn_global_load_lds(kp + goff, (lds_void*)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + goff, (lds_void*)(dst + T::TILE_BYTES), 16, 0, 0);
    }
  };

  // Per-lane pieces of the V transpose-read addresses (see the header comment).
  const int g16 = lane & 15;
  const int gh = (lane >> 4) & 1;
  const int v_row0 = 4 * hh + (g16 >> 2);      // + 32*b + 16*ks2 + 8*r2
  const int v_cpart = 2 * gh + ((g16 & 3) >> 1);  // chunk = 4*db + v_cpart
  const int v_byte = 8 * (g16 & 1);

  fetch(0, 0);
  for (int t = 0; t < ntiles; ++t) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of tile t have landed
    __syncthreads();                 // ... everyone's; and everyone is done with tile t-1
    if (t + 1 < ntiles) fetch(t + 1, (t + 1) & 1);
    const char* kst = smem + (t & 1) * T::STAGE_BYTES;
    const char* vst = kst + T::TILE_BYTES;

    // S^T = K Q^T for the tile: NB blocks of 32 keys x 32 queries.
    f32x16 s[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s[b] = zero16();
      const int row = b * 32 + m32;
      const char* krow = kst + row * T::ROW_BYTES;
      const int sw = swz<D>(row);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 16 * ((2 * kk + hh) ^ sw)));
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

    // P = exp2(S * scale*log2e - m): fp32 for the denominator, bf16 for P V.
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

    // O^T += V^T P^T; the V^T operand comes from two transpose reads per MFMA.
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          s16x4 part[2];
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) {
            const int row = 32 * b + 16 * h2 + 8 * r2 + v_row0;
            const int c = (4 * d + v_cpart) ^ swz<D>(row);
            part[r2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vst + row * T::ROW_BYTES + 16 * c + v_byte));
          }
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
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

template <int D>
hipError_t launch_d(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                    hipStream_t stream) {
  using T = Tile<D>;
  const int QT = int((pr.Nq + T::BM - 1) / T::BM);
  const int64_t n = int64_t(QT) * pr.BH * n_jobs;
  attn_fwd_bf16_kernel<D><<<dim3(unsigned(n)), T::kThreads, 0, stream>>>(
      static_cast<const __bf16*>(q), jobs, pr.Nq, pr.BH, QT, pr.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                            hipStream_t stream) {
  return pr.D == 128 ? launch_d<128>(pr, q, jobs, n_jobs, stream)
                     : launch_d<64>(pr, q, jobs, n_jobs, stream);
}

}  // namespace dita
