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
// * A workgroup owns BM = 4 waves x QB x 32 queries of one (batch, head) and
//   one fresh partition of a grouped launch.  Workgroup ids are remapped so
//   that all query tiles of one (head, partition) run on the same XCD and
//   share its L2 copy of K and V.
// * K and V tiles (BN keys x D) travel HBM -> LDS with direct-to-LDS buffer
//   loads (buffer_load_dwordx4 ... lds): no staging registers, per-lane
//   offsets fixed for the whole kernel, one buffer resource per tile whose
//   records end at the partition end (rows past it read as zero).  In LDS, K
//   rows are padded by 16 bytes and V rows by 64 bytes, which keeps both the
//   K fragment reads and the V transpose reads below free of bank conflicts
//   while every LDS address is one per-lane base plus an immediate.  Padding
//   slots are filled from an offset past the buffer end (zeros, no traffic).
// * Scores are produced transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16: the A operand is a 32-key x 16-dim slice of the
//   K tile, the B operand a 32-query Q^T slice held in registers for the
//   whole kernel.  In the 32x32 accumulator every lane owns ONE query and 16
//   of the 32 keys; its partner lane (lane ^ 32) owns the other 16.  Each K
//   fragment read from LDS feeds QB MFMAs (one per 32-query block).
// * The probabilities feed O^T += V^T P^T directly from registers: for the
//   B operand a lane supplies 8 keys of its own query, and the 8 accumulator
//   entries of one half of an S^T block are exactly that (keys {0-3, 8-11}
//   in the low half-wave, {4-7, 12-15} in the high one).  The matching A
//   operand (8 keys x one head-dim column of V) comes from two LDS transpose
//   reads (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element
//   i%4 of the rows addressed by lanes i/4 + {0,4,8,12}, so pointing lane x
//   at key (x/4) and head-dim offset 4*(x%4) hands every lane 4 keys of its
//   own column.  Each V fragment feeds QB MFMAs.
// * The output accumulator O^T again gives each lane one query, so the
//   online-softmax rescale and the final 1/l are per-lane scalars.  Rescaling
//   is lazy: the running max only moves (and O, l are rescaled) when a
//   tile's max exceeds it by more than 2^8 in the exp2 domain.
// * Tiles run S, softmax, P V in order; the matrix cores and the VALU overlap
//   across the two waves that share each SIMD.  (PIPE, a software pipeline
//   inside each wave -- K one tile ahead of V, the exponentials of tile t
//   beside the S MFMAs of tile t+1 -- measured slower on gfx950 once QB = 2
//   halves the LDS traffic per MFMA: it needs a second S buffer, which costs
//   the second wave per SIMD.)  Measured on the 75,600-token shape: QB=2 and
//   no pipeline 1.03 PFLOP/s, QB=1 with pipeline 0.97, QB=2 with pipeline 0.71.
// * The denominator sums the fp32 probabilities (LSE keeps fp32 accuracy);
//   the P V product uses them rounded to bf16.
// * Ragged tails: query rows past Nq load a clamped row and are not stored;
//   key rows past nk read as zero and their scores are set to -inf.

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

template <int D, int QB>
struct Tile {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BM = kWaves * 32 * QB;        // queries per workgroup
  static constexpr int BN = 4096 / D;                // keys per tile: 32 (D=128), 64 (D=64)
  static constexpr int ROW_BYTES = D * 2;            // one K or V row in HBM
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int KS = ROW_BYTES + 16;          // K row stride in LDS
  static constexpr int VS = ROW_BYTES + 64;          // V row stride in LDS
  static constexpr int K_SPR = KS / 16;              // 16-byte LDS slots per K row
  static constexpr int V_SPR = VS / 16;
  static constexpr int K_REGION = (BN * KS + 1023) / 1024 * 1024;  // whole wave loads
  static constexpr int V_REGION = (BN * VS + 1023) / 1024 * 1024;
  static constexpr int K_WLOADS = K_REGION / 1024;   // wave-wide 16-byte loads per K tile
  static constexpr int V_WLOADS = V_REGION / 1024;
  static constexpr int K_PER_WAVE = (K_WLOADS + kWaves - 1) / kWaves;
  static constexpr int V_PER_WAVE = (V_WLOADS + kWaves - 1) / kWaves;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // bytes of one tile in HBM
  static constexpr int LDS_BYTES = 2 * K_REGION + 2 * V_REGION;
};

// Byte offset, inside a tile in HBM, that fills LDS slot `slot` of a region
// whose rows are `spr` slots long; padding slots get an offset past any
// buffer's end, which the buffer load turns into zeros without a memory access.
__device__ inline uint32_t slot_offset(int slot, int spr, int rows, int cpr, int row_bytes) {
  const int row = slot / spr, col = slot % spr;
  return (row < rows && col < cpr) ? uint32_t(row * row_bytes + col * 16) : 0x7ffffff0u;
}

// One tile HBM -> LDS: wave w issues wave-loads w, w + 4, ...; wave-load i fills
// LDS slots [64 i, 64 i + 64) of `region` (lane-linear), lane data from off[j].
// (A plain device function: the buffer-resource builtins inside a lambda make
// the host pass drop the kernel's launch stub.)
template <int PER_WAVE, int WLOADS>
__device__ inline void load_region(__amdgpu_buffer_rsrc_t r, char* region, int wave,
                                   const uint32_t* off) {
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int i = wave + 4 * j;
    if (i < WLOADS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(region + i * 1024), 16, off[j], 0, 0, 0);
  }
}

// Buffer resource over tile t of one head's K or V: records end at the
// partition end, so rows past nk read as zero.  Every field is made
// explicitly wave-uniform (a resource the compiler cannot prove uniform turns
// each load into a read-first-lane loop).
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const char* head, int t, int tile_bytes,
                                                   uint32_t head_bytes) {
  const uint32_t start = uint32_t(t) * uint32_t(tile_bytes);
  const uint32_t left = head_bytes > start ? head_bytes - start : 0u;
  const uint64_t addr = reinterpret_cast<uint64_t>(head + start);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(addr >> 32));
  const int n = __builtin_amdgcn_readfirstlane(int(left));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, n,
                                           0x00020000);
}

template <typename T>
__device__ inline void load_k_tile(const char* head, int t, uint32_t head_bytes, char* region,
                                   int wave, const uint32_t* off) {
  load_region<T::K_PER_WAVE, T::K_WLOADS>(tile_rsrc(head, t, T::TILE_BYTES, head_bytes), region,
                                          wave, off);
}

template <typename T>
__device__ inline void load_v_tile(const char* head, int t, uint32_t head_bytes, char* region,
                                   int wave, const uint32_t* off) {
  load_region<T::V_PER_WAVE, T::V_WLOADS>(tile_rsrc(head, t, T::TILE_BYTES, head_bytes), region,
                                          wave, off);
}

template <int D, int QB, bool PIPE>
__global__ __launch_bounds__(256, (QB == 2 && PIPE) ? 1 : 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, AttnJobs jobs, int Nq, int BH, int QT, float scale_log2) {
  using T = Tile<D, QB>;
  constexpr int NB = T::BN / 32;   // 32-key blocks per tile
  constexpr int NKK = D / 16;      // MFMA k-steps over the head dim
  constexpr int ND = D / 32;       // 32-wide blocks of the head dim

  // K stage 0, K stage 1, V stage 0, V stage 1.
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  // Workgroup-uniform decode of the tile id (made explicit: integer division is
  // expanded into vector instructions, and values derived from it would
  // otherwise be treated as per-lane).
  const int lin = __builtin_amdgcn_readfirstlane(int(xcd_remap(blockIdx.x, int64_t(gridDim.x))));
  const int qt = __builtin_amdgcn_readfirstlane(lin % QT);
  const int rest = __builtin_amdgcn_readfirstlane(lin / QT);
  const int64_t bh = __builtin_amdgcn_readfirstlane(rest % BH);
  const int jid = __builtin_amdgcn_readfirstlane(rest / BH);

  const AttnJob& job = jobs.job[jid];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31;
  const int hh = lane >> 5;
  const int nk = int(job.nk);
  const int ntiles = (nk + T::BN - 1) / T::BN;

  const uint32_t head_bytes = uint32_t(nk) * T::ROW_BYTES;
  const char* k_head = reinterpret_cast<const char*>(job.k) + bh * int64_t(head_bytes);
  const char* v_head = reinterpret_cast<const char*>(job.v) + bh * int64_t(head_bytes);
  uint32_t k_off[T::K_PER_WAVE], v_off[T::V_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::K_PER_WAVE; ++j)
    k_off[j] = slot_offset((wave + 4 * j) * 64 + lane, T::K_SPR, T::BN, T::CPR, T::ROW_BYTES);
#pragma unroll
  for (int j = 0; j < T::V_PER_WAVE; ++j)
    v_off[j] = slot_offset((wave + 4 * j) * 64 + lane, T::V_SPR, T::BN, T::CPR, T::ROW_BYTES);
  char* const k_stage0 = smem;
  char* const v_stage0 = smem + 2 * T::K_REGION;

  load_k_tile<T>(k_head, 0, head_bytes, k_stage0, wave, k_off);
  if (PIPE && ntiles > 1) load_k_tile<T>(k_head, 1, head_bytes, k_stage0 + T::K_REGION, wave, k_off);
  load_v_tile<T>(v_head, 0, head_bytes, v_stage0, wave, v_off);

  // Q^T operand: for query block qb, lane holds Q[row][kk*16 + 8*hh .. +7].
  const __bf16* __restrict__ qp = q + bh * int64_t(Nq) * D;
  int qrow[QB];
  bf16x8 qf[QB][NKK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = qt * T::BM + (wave * QB + qb) * 32 + m32;
    const int qrow_c = qrow[qb] < Nq ? qrow[qb] : Nq - 1;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[qb][kk] = as_bf16x8(load16(qp + int64_t(qrow_c) * D + kk * 16 + 8 * hh));
  }

  // Per-lane LDS read offsets; everything else is a compile-time immediate.
  //   K fragment (block b, k-step kk): row 32b + m32, bytes [32kk + 16hh, +16).
  //   V transpose read (block b, half h2, read r2, head-dim block d): lane x of a
  //   16-lane group addresses row 32b + 16h2 + 8r2 + 4hh + x/4, head-dim
  //   32d + 16gh + 4(x%4), four elements.
  const int k_lane = m32 * T::KS + 16 * hh;
  const int g16 = lane & 15;
  const int gh = (lane >> 4) & 1;
  const int v_lane = (4 * hh + (g16 >> 2)) * T::VS + 32 * gh + 8 * (g16 & 3);

  f32x16 oacc[QB][ND];
  float m_run[QB], l_run[QB];  // running max (exp2 domain), lane's partial denominator
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[qb][d] = zero16();
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }

  auto compute_s = [&](const char* kreg, f32x16 (*s)[NB]) {
    const char* kb0 = kreg + k_lane;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < NB; ++b) s[qb][b] = zero16();
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const u32x4*>(kb0 + b * 32 * T::KS + 32 * kk));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kk], s[qb][b], 0, 0, 0);
      }
  };
  // Keys past the partition end score -inf (only the last tile has any).
  auto mask_tail = [&](int t, f32x16 (*s)[NB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * T::BN + b * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= nk) s[qb][b][i] = -INFINITY;
        }
  };
  auto row_max = [&](const f32x16 (*s)[NB], float* mx) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, s[qb][b][i]);
      mx[qb] = m;
    }
  };
  // P = exp2(S * scale*log2e - m): fp32 into the denominator, bf16 for P V.
  auto softmax = [&](const f32x16 (*s)[NB], bf16x8 (*pb)[NB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bf16x8 v;
          float part = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float e =
                __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][8 * h2 + j], scale_log2, -m_run[qb]));
            part += e;
            v[j] = (__bf16)e;
          }
          l_run[qb] += part;
          pb[qb][b][h2] = v;
        }
  };
  // O^T += V^T P^T; the V^T operand comes from two transpose reads per MFMA
  // group.  Consecutive MFMAs go to different accumulators.
  auto pv = [&](const char* vreg, bf16x8 (*pb)[NB][2]) {
    const char* vb0 = vreg + v_lane;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          s16x4 part[2];
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2)
            part[r2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vb0 + (32 * b + 16 * h2 + 8 * r2) * T::VS + 64 * d));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][b][h2], oacc[qb][d], 0, 0, 0);
        }
  };
  auto rescale = [&](const float* mx) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m = fmaxf(mx[qb], __shfl_xor(mx[qb], 32));
      const float m_new = fmaxf(m_run[qb], m * scale_log2);
      if (__any(m_new > m_run[qb] + kRescaleSlack)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][d][i] *= alpha;
        m_run[qb] = m_new;
      }
    }
  };

  if constexpr (PIPE) {
    // Start of tile t: wait for K_{t+1} and V_t, free the stages of K_t and
    // V_{t-1}, prefetch K_{t+2} and V_{t+1}, apply the tail mask, update the max.
    auto head = [&](int t, f32x16 (*sc)[NB], float* mx) {
      __builtin_amdgcn_s_waitcnt(0);  // this thread's K_{t+1} and V_t have landed
      __syncthreads();                // ... everyone's; K_t and V_{t-1} are no longer read
      if (t + 2 < ntiles)
        load_k_tile<T>(k_head, t + 2, head_bytes, k_stage0 + (t & 1) * T::K_REGION, wave, k_off);
      if (t + 1 < ntiles)
        load_v_tile<T>(v_head, t + 1, head_bytes, v_stage0 + ((t + 1) & 1) * T::V_REGION, wave,
                       v_off);
      if ((t + 1) * T::BN > nk) {
        mask_tail(t, sc);
        row_max(sc, mx);
      }
      rescale(mx);
    };

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sc[QB][NB];
    float mx[QB];
    compute_s(k_stage0, sc);
    row_max(sc, mx);

    // Tiles with a successor: the exponentials of tile t beside the S MFMAs of
    // tile t+1, the P V MFMAs of tile t beside the row max of tile t+1.
    int t = 0;
    for (; t + 1 < ntiles; ++t) {
      head(t, sc, mx);
      bf16x8 pb[QB][NB][2];
      f32x16 sn[QB][NB];
      softmax(sc, pb);
      compute_s(k_stage0 + ((t + 1) & 1) * T::K_REGION, sn);
      pv(v_stage0 + (t & 1) * T::V_REGION, pb);
      row_max(sn, mx);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int b = 0; b < NB; ++b) sc[qb][b] = sn[qb][b];
    }
    {
      head(t, sc, mx);
      bf16x8 pb[QB][NB][2];
      softmax(sc, pb);
      pv(v_stage0 + (t & 1) * T::V_REGION, pb);
    }
  } else {
    // K_t and V_t share stage t % 2; the next tile is fetched while this one computes.
    for (int t = 0; t < ntiles; ++t) {
      __builtin_amdgcn_s_waitcnt(0);  // this thread's K_t and V_t have landed
      __syncthreads();                // ... everyone's; tile t-1's stage is free
      if (t + 1 < ntiles) {
        load_k_tile<T>(k_head, t + 1, head_bytes, k_stage0 + ((t + 1) & 1) * T::K_REGION, wave,
                       k_off);
        load_v_tile<T>(v_head, t + 1, head_bytes, v_stage0 + ((t + 1) & 1) * T::V_REGION, wave,
                       v_off);
      }
      f32x16 sc[QB][NB];
      float mx[QB];
      compute_s(k_stage0 + (t & 1) * T::K_REGION, sc);
      if ((t + 1) * T::BN > nk) mask_tail(t, sc);
      row_max(sc, mx);
      rescale(mx);
      bf16x8 pb[QB][NB][2];
      softmax(sc, pb);
      pv(v_stage0 + (t & 1) * T::V_REGION, pb);
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (qrow[qb] < Nq) {
      const float inv = 1.0f / l_tot;
      __bf16* __restrict__ op = static_cast<__bf16*>(job.o) + (bh * Nq + qrow[qb]) * int64_t(D);
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)(oacc[qb][d][4 * j + r] * inv);
          *reinterpret_cast<bf16x4*>(op + d * 32 + 8 * j + 4 * hh) = v;
        }
      if (hh == 0) job.lse[bh * Nq + qrow[qb]] = (m_run[qb] + __builtin_log2f(l_tot)) * kLn2;
    }
  }
}

// Tile configuration of the launch: QB query blocks of 32 per wave, and
// whether tiles are software-pipelined inside the wave.
constexpr int kQB = 2;
constexpr bool kPipe = false;

template <int D>
hipError_t launch_d(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                    hipStream_t stream) {
  using T = Tile<D, kQB>;
  const int QT = int((pr.Nq + T::BM - 1) / T::BM);
  const int64_t n = int64_t(QT) * pr.BH * n_jobs;
  attn_fwd_bf16_kernel<D, kQB, kPipe><<<dim3(unsigned(n)), T::kThreads, 0, stream>>>(
      static_cast<const __bf16*>(q), jobs, int(pr.Nq), pr.BH, QT, pr.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                            hipStream_t stream) {
  return pr.D == 128 ? launch_d<128>(pr, q, jobs, n_jobs, stream)
                     : launch_d<64>(pr, q, jobs, n_jobs, stream);
}

}  // namespace dita
