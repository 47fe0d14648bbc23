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
// * A workgroup owns 512 queries (8 waves x 2 blocks of 32) of one (batch,
//   head) and one fresh partition of a grouped launch.  Workgroup ids are
//   remapped so that all query tiles of one (head, partition) run on the same
//   XCD and share its L2 copy of K and V.
// * Ping-pong: the waves form two groups of four (A = waves 0-3, B = 4-7; one
//   wave of each group per SIMD).  Each group alternates an MFMA phase (P V of
//   tile t-1, then S of tile t) with a softmax phase (exponentials of tile t);
//   B runs one phase behind A and one workgroup barrier per tile re-aligns
//   them, so on every SIMD one wave keeps the matrix core busy while the other
//   issues the softmax VALU work.  (A lone wave issues a VALU instruction only every ~6-10
//   cycles on gfx950, so the softmax of a tile takes about as long as its 32
//   MFMAs; left unsynchronised, the two waves of a SIMD drift into the same
//   phase.)
// * Scores are produced transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the A operand is a 32-key x 16-dim slice of the K tile, the B operand a
//   32-query Q^T slice held in registers for the whole kernel.  In the 32x32
//   accumulator every lane owns ONE query and 16 of the 32 keys; its partner
//   lane (lane ^ 32) owns the other 16.  Each K fragment feeds both query
//   blocks of the wave.
// * The probabilities feed O^T += V^T P^T directly from registers: for the B
//   operand a lane supplies 8 keys of its own query, and the 8 accumulator
//   entries of one half of an S^T block are exactly that (keys {0-3, 8-11} in
//   the low half-wave, {4-7, 12-15} in the high one).  The matching A operand
//   (8 keys x one head-dim column of V) comes from two LDS transpose reads
//   (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element i%4
//   of the rows addressed by lanes i/4 + {0,4,8,12}, so pointing lane x at key
//   (x/4) and head-dim offset 4*(x%4) hands every lane 4 keys of its own
//   column.  Each V fragment feeds both query blocks.
// * An MFMA phase is a static schedule of 16 steps (8 P V groups, 8 S k-steps);
//   LDS reads run three steps ahead with explicit lgkmcnt waits.
// * K and V tiles (32 keys x D for D = 128) travel HBM -> LDS with
//   direct-to-LDS buffer loads through a five-stage ring; stage s holds K tile
//   s and V tile s-1, the two operands of MFMA phase s.  (Five, not four: stage
//   t must stay intact through group B's softmax phase of step t, whose rare
//   exact path re-reads K tile t while group A already fetches stage t+4.)  A
//   vector memory instruction occupies the CU's address unit for tens of cycles
//   and stalls its wave meanwhile, so every wave issues exactly two loads per
//   stage, spread over its two phases: its K wave-load at a per-wave step of
//   its MFMA phase, its V wave-load at the start of its softmax phase, two
//   tiles ahead of use.  Rows are stored unpadded (a stage is then
//   16 wave-loads) with the 16-byte chunks of each row permuted by an XOR of
//   the row index, which keeps the K fragment reads and the V transpose reads
//   free of bank conflicts; each read address is a per-lane base XOR a per-step
//   constant plus an immediate.  Rows past the partition end and tiles past
//   the last one are loaded through buffer resources whose records end there
//   (zeros, no memory access).
// * The output accumulator O^T gives each lane one query, so the rescale and
//   the final 1/l are per-lane scalars.  The first tile takes the exact
//   running max; later tiles exponentiate against the running max directly and
//   take the exact max / rescale path (scores recomputed from the K tile still
//   in LDS) only when some lane's partial sum exceeds 2^16, i.e. when a score
//   rose well above the running max.  The denominator sums the fp32
//   probabilities (LSE keeps fp32 accuracy); P V uses them rounded to bf16.
// * Ragged tails: query rows past Nq read as zero (a buffer resource whose
//   records end at Nq) and are not stored; key rows past nk read as zero and
//   their scores are set to -inf.
//
// Measured on one MI355X (4725 x 4725 per head, D = 128, 120 heads): 1.15
// PFLOP/s, against 1.08 for a four-wave kernel without phase synchronisation
// and 1.11 with a barrier between every two phases.

#include "dita_kernels.h"
#include "split_plan.h"
#include "tile_layout.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <utility>

namespace dita {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the running max
constexpr float kFastLimit = 65536.0f; // largest per-lane partial sum the fast path accepts
constexpr int kXcds = 8;

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

// LDS reads issued through inline assembly.  The compiler treats the
// ds_read_b64_tr_b16 builtin as possibly aliasing any pending direct-to-LDS
// buffer load and waits for every outstanding load (the prefetch of later
// stages included) before it; the kernel orders its LDS fills itself (vmcnt
// wait plus barrier before a stage is read), so the reads are issued here and
// their completion is awaited explicitly.  LDS operations complete in order,
// so lgkmcnt(N) with N counting only these reads is exact or waits longer.
__device__ inline uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}
template <int OFF>
__device__ inline s16x4 tr_read(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ inline u32x4 k_read(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// base ^ X computed at this point by one opaque instruction (X = 0: base
// itself): the compiler can neither hoist the result out of the loop (where it
// would hold a register the loop cannot spare) nor copy the base first.
template <int X>
__device__ inline uint32_t xor_here(uint32_t base) {
  if constexpr (X == 0) {
    return base;
  } else {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "n"(X), "v"(base));
    return r;
  }
}

// Wait until at most N LDS operations are outstanding; the fragments are passed
// through so that their consumers cannot be scheduled above the wait.
template <int N>
__device__ inline void lgkm_wait(s16x4& a, s16x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ inline void lgkm_wait1(u32x4& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
// LDS reads still outstanding, in a schedule of steps with PF steps in flight,
// once step i's reads are needed: the reads of steps i+1 .. i+PF-1 (steps below
// NPV issue two reads, the others one).
template <int NPV, int LAST, int PF>
constexpr int pending_reads(int i) {
  int n = 0;
  for (int j = i + 1; j <= i + PF - 1 && j < LAST; ++j) n += j < NPV ? 2 : 1;
  return n;
}

template <int I>
struct Int { static constexpr int value = I; };
template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(Int<I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int D, int QB_ = 2>
struct Tile {
  static constexpr int D_ = D;
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int QB = QB_;                     // 32-query blocks per wave
  static constexpr int BM = kWaves * 32 * QB;        // queries per workgroup
  static constexpr int BN = 4096 / D;                // keys per tile: 32 (D=128), 64 (D=64)
  static constexpr int ROW_BYTES = D * 2;            // one K or V row in HBM
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int K_REGION = BN * ROW_BYTES;   // 8 KB: whole wave-loads, no padding
  static constexpr int V_REGION = BN * ROW_BYTES;
  static constexpr int K_WLOADS = K_REGION / 1024;   // wave-wide 16-byte loads per K tile
  static constexpr int V_WLOADS = V_REGION / 1024;
  static constexpr int WLOADS = K_WLOADS + V_WLOADS;  // per stage: two per wave
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // bytes of one tile in HBM
  static constexpr int STAGE = K_REGION + V_REGION;
  static constexpr int NSTAGE = 5;
  static_assert(K_WLOADS == kWaves && V_WLOADS == kWaves && STAGE % 1024 == 0,
                "one K and one V wave-load per wave and stage");
  // Scratch of one piece of a key-split tile, in the accumulator's register
  // layout (every lane stores and later reloads 16-byte groups of its own
  // registers): the unnormalised O^T accumulators, then per lane the running
  // max and partial denominator of each query block.
  static constexpr int PIECE_O = kWaves * QB * (D / 32) * 4 * 1024;
  static constexpr int PIECE = PIECE_O + kWaves * 1024;
};

// Key-split units of a launch (plan.units == 0: none) and their scratch:
// 2 * units piece slots of Tile<D>::PIECE bytes, and one arrival counter per
// remainder tile, zero before the launch and left zero after it.  A unit's
// range holds at most two segments (it is at most a tile long): the end of the
// tile it starts in and the start of the next one; one workgroup computes both,
// one after the other.
struct SplitArgs {
  SplitPlan plan;
  char* pieces;
  int* count;
};
constexpr int kMaxPieces = kSplitMaxPieces;

// Per-workgroup state of a split segment, in LDS rather than in scalar
// registers: nothing of it stays live through the tile's main loop (the
// epilogue reads it back after the loop's barriers).
struct SplitShared {
  SplitPlan plan;
  char* pieces;
  int* count;
  int64_t unit;
  int64_t r;       // remainder tile of this segment if it is a piece, else -1
  int arrived;     // arrivals counted before this workgroup's piece
};
__device__ inline SplitShared* split_shared() {
  __shared__ SplitShared sh;
  return &sh;
}
template <typename V>
__device__ inline V uniform_lds(const V& v) {
  if constexpr (sizeof(V) == 8) {
    const int64_t w = __builtin_bit_cast(int64_t, v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(w));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(w) >> 32));
    return __builtin_bit_cast(V, int64_t((uint64_t(hi) << 32) | lo));
  } else {
    return __builtin_bit_cast(V, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
  }
}

// LDS layout of a K or V tile: rows of ROW_BYTES, unpadded, with the 16-byte
// chunks of each row permuted by an XOR of the row index (physical chunk =
// logical chunk ^ f(row)).  On gfx950 the LDS serves ds_read_b128 16 lanes at a
// time and ds_read_b64_tr_b16 32 lanes at a time over 64 four-byte banks; a
// pattern is conflict-free when the lanes of one pass hit distinct 16-byte
// (resp. 8-byte) slots modulo 256 bytes (measured: the padded strides that meet
// this read with zero SQ_LDS_BANK_CONFLICT).  K fragment reads take one chunk
// from 16 consecutive rows; transpose reads take two adjacent chunks and both
// 8-byte halves from 4 consecutive rows, for two 32-byte column groups.
//   D = 128 (16 chunks per row): f_K(r) = r & 15,        f_V(r) = 4 (r & 3)
//   D = 64  (8 chunks per row):  f_K(r) = (r >> 1) & 7, f_V(r) = 4 ((r >> 1) & 1)
template <int D>
__device__ inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Byte offset, inside a tile in HBM, of the 16 bytes that land in LDS slot
// `slot` (16-byte units, row-major) of a K (IS_K) or V region.
template <typename T, bool IS_K>
__device__ inline uint32_t swz_offset(int slot) {
  const int row = slot / T::CPR, phys = slot % T::CPR;
  const int chunk = phys ^ (IS_K ? swz_k<T::D_>(row) : swz_v<T::D_>(row));
  return uint32_t(row * T::ROW_BYTES + chunk * 16);
}

// Buffer resource over tile t of one head's K or V: records end at the
// partition end, so rows past nk (and every tile at or past the last one) read
// as zero.  Every field is made explicitly wave-uniform (a resource the
// compiler cannot prove uniform turns each load into a read-first-lane loop).
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const char* head, int t, int tile_bytes,
                                                   uint32_t head_bytes) {
  const uint32_t start = __builtin_amdgcn_readfirstlane(uint32_t(t) * uint32_t(tile_bytes));
  const uint32_t hb = __builtin_amdgcn_readfirstlane(head_bytes);
  // max(head_bytes - start, 0) on the scalar unit (written out: the compiler's
  // saturating subtraction is a vector instruction plus a read-back)
  uint32_t left;
  asm("s_sub_u32 %0, %1, %2\n\ts_cselect_b32 %0, 0, %0" : "=s"(left) : "s"(hb), "s"(start) : "scc");
  const uint64_t addr = reinterpret_cast<uint64_t>(head + start);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(addr >> 32));
  const int n = int(left);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, n,
                                           0x00020000);
}

// Load J (0 or 1) of a wave's share of stage s: wave w fills K wave-load w
// (J = 0) and V wave-load w (J = 1) of the stage, K tile s and V tile s-1,
// with per-lane source offsets fixed for the whole kernel (off_k, off_v).
// Stage 0 has no V tile: its V loads use the empty tile past the end, so every
// wave issues the same two loads for every stage.  (A plain device function:
// buffer-resource builtins inside a kernel lambda make the host pass drop the
// launch stub.)
template <typename T, int J>
__device__ inline void load_share_item(char* smem, int s, int ntiles, const char* k_head,
                                       const char* v_head, uint32_t head_bytes, int wave,
                                       uint32_t off_k, uint32_t off_v) {
  char* base = smem + (s % T::NSTAGE) * T::STAGE;
  if constexpr (J == 0) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(k_head, s, T::TILE_BYTES, head_bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(base + wave * 1024), 16, off_k, 0,
                                             0, 0);
  } else {
    const __amdgpu_buffer_rsrc_t rv =
        tile_rsrc(v_head, s >= 1 ? s - 1 : ntiles, T::TILE_BYTES, head_bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(base + T::K_REGION + wave * 1024),
                                             16, off_v, 0, 0, 0);
  }
}
// vmcnt waits.  Every wave issues the same loads for every stage (a K and a V
// load, or two of each for DUAL tiles); the wait leaves exactly STAGES later
// stages plus the K loads of EXTRA stages in flight.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt(N), expcnt and lgkmcnt not waited for
}
template <int STAGES, int EXTRA, bool DUAL = false>
__device__ inline void wait_stages_in_flight() {
  // DUAL tiles: each wave issues two K and two V loads per stage (EXTRA counts
  // the K loads of one stage).
  wait_vm<(DUAL ? 4 : 2) * STAGES + (DUAL ? 2 : 1) * EXTRA>();
}
__device__ inline void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier without a memory fence: LDS contents are ordered by the
// explicit vmcnt waits of the waves that loaded them.
__device__ inline void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kCoherent = 16;  // buffer cache policy: sc1 (agent scope)
// Bit casts through by-value parameters (a bit cast of a vector-element lvalue
// reads element 0).
__device__ inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ inline float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// The tile's output from its n pieces (2 <= n <= NP) in scratch slots
// slot[0 .. n-1] (key order): weights from the pieces' running maxima, then
// per 16-byte group of accumulators the weighted sum, normalised, rounded to
// bf16 and stored; the loads of G groups of all pieces are issued before any
// is used (the registers of a batch hold G * NP groups; G divides the 16
// groups of a lane's accumulators).
template <int D, int NP, int G>
__device__ __forceinline__ void split_combine(__amdgpu_buffer_rsrc_t rs, const uint32_t (&slot)[kMaxPieces],
                                              int n, int wave, int lane, const int (&qrow)[2], int Nq,
                                              __bf16* o_head, float* lse_head) {
  using T = Tile<D, 2>;
  constexpr int ND = D / 32;
  static_assert(NP <= kMaxPieces, "pieces");
  const uint32_t lane_off = uint32_t(lane) * 16;
  const uint32_t stats_off = uint32_t(T::PIECE_O + wave * 1024) + lane_off;
  float ms[NP][2], ls[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ms[i][0] = ms[i][1] = -INFINITY;
    ls[i][0] = ls[i][1] = 0.0f;
    if (i < n) {
      const u32x4 st = __builtin_amdgcn_raw_buffer_load_b128(rs, stats_off, slot[i], kCoherent);
      ms[i][0] = u2f(st[0]);
      ls[i][0] = u2f(st[1]);
      ms[i][1] = u2f(st[2]);
      ls[i][1] = u2f(st[3]);
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = ms[0][qb];
#pragma unroll
    for (int i = 1; i < NP; ++i) mx = fmaxf(mx, ms[i][qb]);
    float w[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) w[i] = __builtin_amdgcn_exp2f(ms[i][qb] - mx);
    float l = w[0] * ls[0][qb];
#pragma unroll
    for (int i = 1; i < NP; ++i)
      if (i < n) l = __builtin_fmaf(w[i], ls[i][qb], l);
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = 1.0f / l_tot;
    const bool valid = qrow[qb] < Nq;
    __bf16* __restrict__ op = o_head + int64_t(valid ? qrow[qb] : 0) * D;
    const uint32_t base = uint32_t(((wave * 2 + qb) * ND * 4) * 64 * 16) + lane_off;
    for (int c0 = 0; c0 < ND * 4; c0 += G) {
      u32x4 x[G][NP];
#pragma unroll
      for (int i = 0; i < NP; ++i)
        if (i < n) {
#pragma unroll
          for (int g = 0; g < G; ++g)
            x[g][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + uint32_t((c0 + g) * 1024),
                                                            slot[i], kCoherent);
        }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w[0] * u2f(x[g][0][e]);
#pragma unroll
        for (int i = 1; i < NP; ++i)
          if (i < n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w[i], u2f(x[g][i][e]), acc[e]);
          }
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[e] * inv);
        const int c = c0 + g, d = c >> 2, j = c & 3;
        if (valid) *reinterpret_cast<bf16x4*>(op + d * 32 + 8 * j + 4 * (lane >> 5)) = v;
      }
    }
    if (valid && lane < 32) lse_head[qrow[qb]] = (mx + __builtin_log2f(l_tot)) * kLn2;
  }
}

// Pieces of a key-split tile (QB = 2).  Every piece stores its unnormalised
// state; the piece that arrives last at the tile's counter reloads all of them
// (its own included) and writes the tile's output: the weighted sum over the
// pieces in key order, one 16-byte group of accumulators at a time.  Every
// value is read from the scratch, so the result does not depend on which piece
// finished last.
//
// Ordering across XCDs (each has its own L2) without whole-cache fences: the
// piece is stored and reloaded with agent-scope coherent accesses (the sc1
// cache policy, the encoding of agent-scope atomic stores and loads); every
// wave waits for its stores to complete before the workgroup barrier after
// which one thread increments the tile's counter (an agent-scope atomic); the
// combining workgroup issues its reloads only after that increment returned.
// A completed coherent store is visible to every later coherent load, and the
// counter's increments are totally ordered, so the last piece sees all others.
// It resets the counter to zero for the next launch.  (Agent-scope release
// and acquire fences would write back and invalidate the whole L2 of the XCD
// for every piece, under the other workgroups' K/V tiles: measured 4-9% slower
// launches than these per-access scopes.)
template <int D>
__device__ __forceinline__ void split_piece(const f32x16 (&oacc)[2][D / 32], const float (&m_run)[2],
                                            const float (&l_run)[2], int64_t r, int wave, int lane,
                                            const int (&qrow)[2], int Nq, __bf16* o_head,
                                            float* lse_head) {
  using T = Tile<D, 2>;
  constexpr int ND = D / 32;
  SplitShared* sh = split_shared();
  SplitPlan p;
  p.units = uniform_lds(sh->plan.units);
  p.rem = uniform_lds(sh->plan.rem);
  p.T = uniform_lds(sh->plan.T);
  p.G = uniform_lds(sh->plan.G);
  char* const pieces = uniform_lds(sh->pieces);
  int* const count = uniform_lds(sh->count);
  const int64_t unit = uniform_lds(sh->unit);
  // One buffer resource over all 2U slots (< 2^32 bytes); a slot is the scalar offset.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      pieces, 0, int(uint32_t(2 * p.units) * uint32_t(T::PIECE)), 0x00020000);
  const uint32_t lane_off = uint32_t(lane) * 16;
  auto chunk_off = [&](int qb, int c) {
    return uint32_t((((wave * 2 + qb) * ND * 4 + c) * 64) * 16) + lane_off;
  };
  const uint32_t stats_off = uint32_t(T::PIECE_O + wave * 1024) + lane_off;
  auto slot_base = [&](int64_t u) {
    return __builtin_amdgcn_readfirstlane(uint32_t(split_slot(p, u, r)) * uint32_t(T::PIECE));
  };

  const uint32_t own = slot_base(unit);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f2u(oacc[qb][d][4 * j + e]);
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, chunk_off(qb, d * 4 + j), own, kCoherent);
      }
  {
    u32x4 v;
    v[0] = f2u(m_run[0]);
    v[1] = f2u(l_run[0]);
    v[2] = f2u(m_run[1]);
    v[3] = f2u(l_run[1]);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, stats_off, own, kCoherent);
  }
  wait_loads();  // vmcnt(0): this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    sh->arrived = __hip_atomic_fetch_add(count + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int n = split_pieces(p, r);
  if (uniform_lds(sh->arrived) != n - 1) return;
  if (threadIdx.x == 0) __hip_atomic_store(count + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const int64_t first = split_first_unit(p, r);
  uint32_t slot[kMaxPieces];
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) slot[i] = slot_base(first + (i < n ? i : 0));
  // Two 16-byte groups of every piece per batch of loads: a batch of all
  // kMaxPieces pieces then holds 64 registers (four groups spill).
  split_combine<D, kMaxPieces, 2>(rs, slot, n, wave, lane, qrow, Nq, o_head, lse_head);
}

// One query tile: QB * 256 query rows from row0 of head bh against job jid's
// partition (QB = 2: 512-row tiles; QB = 1: 256-row tiles for the tail rows),
// over the partition's key tiles [kt0, kt1) (kt1 < 0: to the end).  A 512-row
// tile whose split state (LDS) names a remainder tile is a piece of it.
// DUAL (QB = 1): the two wave groups take the tails of two (head, block)
// pairs, (jid, bh, row0) for waves 0-3 and (jid_b, bh_b, row0_b) for waves
// 4-7, 128 rows each, each group with its own LDS ring of K/V stages that its
// four waves fill (two K and two V chunks each per stage).  Both pairs must
// have the same number of keys (the groups share the per-tile barriers).
template <int D, int QB, bool SPLIT = false, int SEG = 0, bool DUAL = false>
__device__ __forceinline__ void attn_tile(char* smem_base, const __bf16* __restrict__ q,
                                          const AttnJobs& jobs, int jid_a, int64_t bh_a,
                                          int64_t row0_a, int Nq, float scale_log2, int kt0 = 0,
                                          int kt1 = -1, int jid_b = 0, int64_t bh_b = 0,
                                          int64_t row0_b = 0) {
  using T = Tile<D, QB>;
  constexpr int NB = T::BN / 32;
  constexpr int NKK = D / 16;
  constexpr int ND = D / 32;
  static_assert(!DUAL || QB == 1, "dual tiles are 256-row tiles");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wl = wave & 3;
  const bool second = DUAL && grp == 1;  // wave-uniform
  const int jid = second ? jid_b : jid_a;
  const int64_t bh = second ? bh_b : bh_a;
  const int64_t row0 = second ? row0_b : row0_a;
  char* const smem = DUAL ? smem_base + grp * (T::NSTAGE * T::STAGE) : smem_base;
  const AttnJob& job = jobs.job[jid];
  // First query block of this wave in its tile, and the tile's rows.
  const int qblk0 = DUAL ? wl * QB : wave * QB;
  constexpr int BMW = DUAL ? 4 * 32 * QB : T::BM;
  const int m32 = lane & 31;
  const int hh = lane >> 5;
  // Keys of this tile: all of the partition's, or (split launches) its key
  // tiles [kt0, kt1) (kt1 < 0: to the end).
  int nk, ntiles;
  int64_t key_off;
  if constexpr (SPLIT) {
    const int nk_all = int(job.nk);
    const int kt_end = kt1 < 0 ? (nk_all + T::BN - 1) / T::BN : kt1;
    nk = min(nk_all - kt0 * T::BN, (kt_end - kt0) * T::BN);
    ntiles = kt_end - kt0;
    key_off = bh * int64_t(nk_all) * T::ROW_BYTES + int64_t(kt0) * T::TILE_BYTES;
  } else {
    nk = int(job.nk);
    ntiles = (nk + T::BN - 1) / T::BN;
    key_off = bh * int64_t(uint32_t(nk) * T::ROW_BYTES);
  }

  const uint32_t head_bytes = uint32_t(nk) * T::ROW_BYTES;
  // The 1 KB chunks of a stage's K and V regions this wave fills: chunk `wave`
  // of each, or (DUAL) chunks wl and wl + 4 of its group's ring.
  const int ck0 = DUAL ? wl : wave;
  const int ck1 = wl + 4;
  const uint32_t off_k = swz_offset<T, true>(ck0 * 64 + lane);
  const uint32_t off_v = swz_offset<T, false>(ck0 * 64 + lane);
  const uint32_t off_k1 = DUAL ? swz_offset<T, true>(ck1 * 64 + lane) : 0u;
  const uint32_t off_v1 = DUAL ? swz_offset<T, false>(ck1 * 64 + lane) : 0u;
  const char* k_head = reinterpret_cast<const char*>(job.k) + key_off;
  const char* v_head = reinterpret_cast<const char*>(job.v) + key_off;
  const __bf16* __restrict__ qp = q + bh * int64_t(Nq) * D;
  int qrow[QB];
  bf16x8 qf[QB][NKK];
  // Q of this query tile through a buffer resource whose records end at row Nq:
  // rows past it read as zero, so their (discarded) MFMAs multiply zeros.
  const int64_t tile_row0 = row0;
  const int64_t rows_left = int64_t(Nq) - tile_row0;
  const __amdgpu_buffer_rsrc_t rq =
      tile_rsrc(reinterpret_cast<const char*>(qp + tile_row0 * D), 0, 0,
                uint32_t((rows_left < 0 ? 0 : rows_left < BMW ? rows_left : BMW) * D * 2));
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = int(row0) + (qblk0 + qb) * 32 + m32;
    const int lrow = (qblk0 + qb) * 32 + m32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[qb][kk] = as_bf16x8(__builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rq, uint32_t(lrow * D * 2 + (kk * 16 + 8 * hh) * 2), 0, 0)));
  }
  auto load_k = [&](int st) {
    load_share_item<T, 0>(smem, st, ntiles, k_head, v_head, head_bytes, ck0, off_k, off_v);
    if constexpr (DUAL)
      load_share_item<T, 0>(smem, st, ntiles, k_head, v_head, head_bytes, ck1, off_k1, off_v1);
  };
  auto load_v = [&](int st) {
    load_share_item<T, 1>(smem, st, ntiles, k_head, v_head, head_bytes, ck0, off_k, off_v);
    if constexpr (DUAL)
      load_share_item<T, 1>(smem, st, ntiles, k_head, v_head, head_bytes, ck1, off_k1, off_v1);
  };
#pragma unroll
  for (int st0 = 0; st0 < 3; ++st0) {
    load_k(st0);
    load_v(st0);
  }

  // Per-lane LDS offsets inside a stage; a step adds an immediate and XORs a
  // constant into bits the lane part leaves clear (the stage base is 1 KB aligned):
  //   K fragment (block b, k-step kk): (k_lane ^ 32 kk) + 32 b ROW_BYTES
  //   V transpose read (block b, half h2, read r2, head-dim block d):
  //     (v_lane ^ 64 d) + (32 b + 16 h2 + 8 r2) ROW_BYTES
  const int k_lane = m32 * T::ROW_BYTES + 16 * (hh ^ swz_k<D>(m32));
  const int g16 = lane & 15;
  const int gh = (lane >> 4) & 1;
  const int vrow = 4 * hh + (g16 >> 2);
  const int v_lane = vrow * T::ROW_BYTES + 32 * gh + 8 * (g16 & 3) + 16 * swz_v<D>(vrow);

  f32x16 oacc[QB][ND];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[qb][d] = zero16();
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }

  auto compute_s = [&](const char* kreg, f32x16 (*s)[NB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < NB; ++b) s[qb][b] = zero16();
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const u32x4*>(kreg + (k_lane ^ (32 * kk)) + b * 32 * T::ROW_BYTES));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kk], s[qb][b], 0, 0, 0);
      }
  };
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
  // Eight exponentials against the running max (bf16 copies for P V) and
  // their fp32 sum as a pairwise tree (depth 3 instead of a chain of 8).
  auto exp8 = [&](const f32x16& s, int h2, float m, bf16x8& v) -> float {
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h2 + j], scale_log2, -m));
      v[j] = (__bf16)e[j];
    }
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  };
  // Sum of the exponentials of one query block's 16 x NB scores of this lane.
  auto exp_block = [&](int qb, const f32x16 (*s)[NB], bf16x8 (*pb)[NB][2]) -> float {
    float part = exp8(s[qb][0], 0, m_run[qb], pb[qb][0][0]);
    part += exp8(s[qb][0], 1, m_run[qb], pb[qb][0][1]);
#pragma unroll
    for (int b = 1; b < NB; ++b) {
      part += exp8(s[qb][b], 0, m_run[qb], pb[qb][b][0]);
      part += exp8(s[qb][b], 1, m_run[qb], pb[qb][b][1]);
    }
    return part;
  };
  // Exponentials of one query block against the running max, fp32 sum into
  // the lane's partial denominator, bf16 copies for P V.
  auto softmax_qb = [&](int qb, const f32x16 (*s)[NB], bf16x8 (*pb)[NB][2]) {
    l_run[qb] += exp_block(qb, s, pb);
  };
  auto softmax = [&](const f32x16 (*s)[NB], bf16x8 (*pb)[NB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) softmax_qb(qb, s, pb);
  };
  auto rescale_qb = [&](int qb, float mxq) {
    const float m = fmaxf(mxq, __shfl_xor(mxq, 32));
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
  };
  auto rescale = [&](const float* mx) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rescale_qb(qb, mx[qb]);
  };
  // Exponentials against the running max, without a tile max (after the first
  // tile the running max is finite).  Returns false, leaving l untouched, if
  // some lane's partial sum exceeds 2^16 or is not finite; the caller then
  // takes the exact max / rescale path.  Masked keys (-inf) give exactly 0 on
  // either path.  `between(qb)` runs before each query block (load issue).
  auto softmax_fast = [&](const f32x16 (*s)[NB], bf16x8 (*pb)[NB][2], auto&& between) -> bool {
    float part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      between(qb);
      part[qb] = exp_block(qb, s, pb);
    }
    uint64_t bad = 0;  // lanes whose partial sum is too large or not finite
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bad |= __builtin_amdgcn_ballot_w64(!(part[qb] <= kFastLimit));
    const bool all_ok = bad == 0;  // wave-uniform
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += all_ok ? part[qb] : 0.0f;
    return all_ok;
  };

  // One MFMA phase as a static schedule of steps: steps [0, NPV) are the P V
  // groups of the previous tile (two transpose reads, QB MFMAs each), steps
  // [NPV, NPV + NS) the S k-steps of this tile (one K read, QB MFMAs each).
  // Reads run PF steps ahead of their MFMAs.
  constexpr int NPV = NB * 2 * ND;
  constexpr int NS = NB * NKK;
  constexpr int PF = 3;
  auto m_phase = [&](auto first_c, auto last_c, const char* stg, f32x16 (*s)[NB],
                     bf16x8 (*pb)[NB][2], int load_stage_idx) {
    constexpr int FIRST = decltype(first_c)::value;
    constexpr int LAST = decltype(last_c)::value;
    const uint32_t va = lds_addr(stg + T::K_REGION + v_lane);
    const uint32_t ka = lds_addr(stg + k_lane);
    s16x4 fr[NPV][2];
    u32x4 kf[NS];
    auto issue = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < NPV) {
        constexpr int b = i / (2 * ND), h2 = (i / ND) % 2, d = i % ND;
        const uint32_t a = xor_here<64 * d>(va);
        fr[i][0] = tr_read<(32 * b + 16 * h2) * T::ROW_BYTES>(a);
        fr[i][1] = tr_read<(32 * b + 16 * h2 + 8) * T::ROW_BYTES>(a);
      } else {
        constexpr int j = i - NPV, b = j / NKK, kk = j % NKK;
        kf[j] = k_read<b * 32 * T::ROW_BYTES>(xor_here<32 * kk>(ka));
      }
    };
    static_for<PF>([&](auto c) {
      constexpr int i = FIRST + decltype(c)::value;
      if constexpr (i < LAST) issue(Int<i>{});
    });
    static_for<LAST - FIRST>([&](auto c) {
      constexpr int i = FIRST + decltype(c)::value;
      constexpr int pend = pending_reads<NPV, LAST, PF>(i);
      if constexpr (i < NPV) {
        constexpr int b = i / (2 * ND), h2 = (i / ND) % 2, d = i % ND;
        lgkm_wait<pend>(fr[i][0], fr[i][1]);
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(fr[i][0], fr[i][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][b][h2], oacc[qb][d], 0, 0, 0);
      } else {
        constexpr int j = i - NPV, b = j / NKK, kk = j % NKK;
        lgkm_wait1<pend>(kf[j]);
        const bf16x8 a = as_bf16x8(kf[j]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kk],
                                                             kk == 0 ? zero16() : s[qb][b], 0, 0, 0);
      }
      if constexpr (i + PF < LAST) issue(Int<i + PF>{});
      // Item 0 of this wave's share of stage load_stage_idx, at a step that
      // differs per wave of the group (staggered use of the address unit).
      if constexpr ((i - FIRST) % 4 == 1 && (i - FIRST) / 4 < 4) {
        if (load_stage_idx >= 0 && wl == (i - FIRST) / 4) load_k(load_stage_idx);
      }
      // Keep the written order: each step's MFMAs before the next step's wait.
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Phase schedule (group A = waves 0-3, B = waves 4-7), one barrier per tile:
  //   A: M(t) V(t) | M(t+1) V(t+1) | ...      B: M(t) | V(t) M(t+1) | ...
  // M(t) = P V of tile t-1 and S of tile t, reading stage t; V(t) = softmax of
  // tile t.  The barrier after A's V(t) and B's M(t) re-aligns the groups every
  // tile, so A's MFMA phase runs beside B's softmax phase and the other way
  // round (B starts one phase late: its first M overlaps A's first two).
  // Every wave fetches its two loads of stage t+3 during M(t) (the K load, at a
  // step that differs per wave) and V(t) (the V load); its share of stage s has
  // landed at the barrier that ends tile s-1: group A waits at the end of
  // V(s-1) with stages s+1, s+2 in flight, group B at the end of M(s-1) with
  // stage s+1 and the K load of stage s+2 in flight.  Stage t is rewritten by
  // stage t+5, whose first load A issues after the barrier that ends tile t+1,
  // when B's softmax of tile t (whose exact path may re-read K tile t) is done.
  wait_stages_in_flight<2, 0, DUAL>();  // stage 0 (stages 1, 2 in flight)
  phase_barrier();
  // A wave whose query blocks all lie past Nq (the padding rows of a tail
  // tile) computes nothing: under the board's power cap its MFMAs and
  // exponentials would only lower the clock of the waves that do.  It keeps
  // its share of every stage's loads, in the same order, and takes every
  // barrier of the schedule below, then leaves (its rows are not stored).
  // Split launches, whose pieces meet at further barriers, keep every wave.
  if constexpr (!SPLIT) {
    if (row0 + int64_t(qblk0) * 32 >= Nq) {  // wave-uniform
      for (int t = 0; t < ntiles; ++t) {
        load_k(t + 3);
        if (grp == 1) {
          wait_stages_in_flight<1, 1, DUAL>();
          phase_barrier();
        }
        load_v(t + 3);
        if (grp == 0) {
          wait_stages_in_flight<2, 0, DUAL>();
          phase_barrier();
        }
      }
      wait_loads();
      return;
    }
  }
  f32x16 sc[QB][NB];
  bf16x8 pb[QB][NB][2];
  if (ntiles > 0) {  // step 0: S only, exact max
    __builtin_amdgcn_s_setprio(1);
    m_phase(Int<NPV>{}, Int<NPV + NS>{}, smem, sc, pb, 3);
    if (wl >= 2) load_k(3);
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) {
      wait_stages_in_flight<1, 1, DUAL>();
      phase_barrier();
    }
    load_v(3);
    if (T::BN > nk) mask_tail(0, sc);
    float mx[QB];
    row_max(sc, mx);
    rescale(mx);
    softmax(sc, pb);
    if (grp == 0) {
      wait_stages_in_flight<2, 0, DUAL>();
      phase_barrier();
    }
  }
  for (int t = 1; t < ntiles; ++t) {
    const char* st = smem + (t % T::NSTAGE) * T::STAGE;
    __builtin_amdgcn_s_setprio(1);
    m_phase(Int<0>{}, Int<NPV + NS>{}, st, sc, pb, t + 3);
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) {
      wait_stages_in_flight<1, 1, DUAL>();
      phase_barrier();
    }

    if ((t + 1) * T::BN > nk) mask_tail(t, sc);
    // The V load goes ahead of the first query block (measured faster than
    // placing it between the blocks for half of the waves).
    auto loads_between = [&](int qb) {
      __builtin_amdgcn_sched_barrier(0);
      if (qb == 0) load_v(t + 3);
      __builtin_amdgcn_sched_barrier(0);
    };
    const bool fast = softmax_fast(sc, pb, loads_between);
    if (!fast) {
      // The fast path consumed the scores: recompute them from the K tile.
      compute_s(smem + (t % T::NSTAGE) * T::STAGE, sc);
      if ((t + 1) * T::BN > nk) mask_tail(t, sc);
      float mx[QB];
      row_max(sc, mx);
      rescale(mx);
      softmax(sc, pb);
    }
    if (grp == 0) {
      wait_stages_in_flight<2, 0, DUAL>();
      phase_barrier();
    }
  }
  if (ntiles > 0) {
    __builtin_amdgcn_s_setprio(1);
    m_phase(Int<0>{}, Int<NPV>{}, smem + (ntiles % T::NSTAGE) * T::STAGE, sc, pb, -1);
    __builtin_amdgcn_s_setprio(0);
  }
  wait_loads();  // the zero-filling loads past the last stage must land before LDS is released

  // Split launches: lane indices of the epilogue derived anew behind an opaque
  // copy (values computed from them are not kept live from the first segment
  // into the second), and pieces of split tiles handled here.
  int lane_e = lane, hh_e = hh, qrow_e[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qrow_e[qb] = qrow[qb];
  if constexpr (SPLIT && QB == 2) {
    int tid_e = int(threadIdx.x);
    asm volatile("" : "+v"(tid_e));
    lane_e = tid_e & 63;
    hh_e = lane_e >> 5;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qrow_e[qb] = int(row0) + (qblk0 + qb) * 32 + (lane_e & 31);
    const int64_t piece_r = uniform_lds(split_shared()->r);
    if (piece_r >= 0) {
      split_piece<D>(oacc, m_run, l_run, piece_r, wave, lane_e, qrow_e, Nq,
                     static_cast<__bf16*>(job.o) + bh * Nq * int64_t(D), job.lse + bh * Nq);
      return;
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (qrow_e[qb] < Nq) {
      const float inv = 1.0f / l_tot;
      __bf16* __restrict__ op = static_cast<__bf16*>(job.o) + (bh * Nq + qrow_e[qb]) * int64_t(D);
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)(oacc[qb][d][4 * j + r] * inv);
          *reinterpret_cast<bf16x4*>(op + d * 32 + 8 * j + 4 * hh_e) = v;
        }
      if (hh_e == 0) job.lse[bh * Nq + qrow_e[qb]] = (m_run[qb] + __builtin_log2f(l_tot)) * kLn2;
    }
  }
}

// Query tiles of one (head, block): `big` 512-row tiles from row 0, then
// `small` 256-row tiles.
struct TileSplit {
  int big;
  int small;
};

// Time of a 256-row workgroup holding the tails (<= 128 rows each) of two
// (head, block) pairs, relative to a 512-row tile (from the measured gain of
// the 16-block launches at the 75,600-token shape: 1.3% against 2.1% for
// 0.70; each wave loads twice the K/V of a single tail per key tile).
constexpr double kDualTileCost = 0.85;

// (estimated_makespan models the 256-row tiles dispatched after all 512-row
// tiles.  The interleaved layout dispatches each (head, block)'s 256-row tiles
// right after its 512-row ones instead, so that they share the block's K/V in
// L2: measured at the same launch times as dispatching them last, with 1.5 GB
// less HBM traffic per 16-block launch at the 75,600-token shape.)

// The rows past the last whole 512-row tile (4725 = 9 * 512 + 117 rows at the
// 75,600-token shape) go either into one more 512-row tile or into 256-row
// tiles, whichever the estimate above finishes first for `per` (head, block)
// pairs on `cus` compute units.  (Measured: moving more rows than these into
// 256-row tiles in this per-pair order makes launches slower, not faster: the
// 512-row tiles then spread over more rounds than the estimate assumes.  The
// staged layout moves more rows into 256-row tiles, dispatched after all
// 512-row tiles.)
TileSplit choose_tile_split(int64_t Nq, int64_t per, int cus) {
  const int whole = int(Nq / 512), all_big = int((Nq + 511) / 512);
  const TileSplit big_only{all_big, 0};
  if (whole == all_big) return big_only;
  const TileSplit with_small{whole, int((Nq - int64_t(whole) * 512 + 255) / 256)};
  const double t_big = estimated_makespan(int64_t(all_big) * per, 0, cus, kSmallTileCost);
  const double t_small = estimated_makespan(int64_t(whole) * per, int64_t(with_small.small) * per,
                                            cus, kSmallTileCost);
  return t_small < t_big - 1e-9 ? with_small : big_only;
}

// Compute units of the current device (looked up once per device).
hipError_t compute_units(int* cus, int* device = nullptr) {
  static int cached[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (device) *device = dev;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) {
    *cus = cached[dev];
    return hipSuccess;
  }
  int n = 0;
  if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  *cus = n;
  return hipSuccess;
}

// Grid: per (head, block) in linear order, QT_big 512-row tiles then QT_small
// 256-row tiles (the rows after the 512-row tiles), n_big + n_small in all,
// remapped so that all tiles of one (head, block) land on one XCD; then (SPLIT
// instantiation, no 256-row tiles) sa.plan.units key-split units, which share
// the last sa.plan.rem 512-row tiles in linear order, [n_big, n_big + rem).
// Launches without split units use the other instantiation, which carries
// none of the split's code.
// Staged layout (stage_a >= 0, no split units, no dual tails): all n_big
// 512-row tiles first, then all n_small 256-row tiles, each kind remapped by
// itself; pairs [0, stage_a) have QT_big 512-row and QT_small 256-row tiles,
// the others QT_big - 1 and QT_small_b.
template <int D, bool SPLIT, bool DUAL = false>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, AttnJobs jobs, int Nq, int BH, int n_big, int QT_big,
    int n_small, int QT_small, SplitArgs sa, float scale_log2, int pairs, int stage_a,
    int QT_small_b) {
  __shared__ __attribute__((aligned(1024)))
  char smem[(DUAL ? 2 : 1) * Tile<D>::NSTAGE * Tile<D>::STAGE];
  const int pid = blockIdx.x;
  if constexpr (DUAL) {
    // Per two (head, block) pairs: the first's 512-row tiles, the second's,
    // then one workgroup for both pairs' tail rows (at most 128 each); an odd
    // last pair shares its tail workgroup with no rows.
    const int per_unit = 2 * QT_big + 1;
    const int lin = __builtin_amdgcn_readfirstlane(int(xcd_remap(pid, n_big + n_small)));
    const int pp = __builtin_amdgcn_readfirstlane(lin / per_unit);
    const int j = __builtin_amdgcn_readfirstlane(lin % per_unit);
    const bool has_b = 2 * pp + 1 < pairs;
    if (j < (has_b ? 2 * QT_big : QT_big)) {
      const int pair = __builtin_amdgcn_readfirstlane(2 * pp + (j >= QT_big ? 1 : 0));
      const int qt = __builtin_amdgcn_readfirstlane(j >= QT_big ? j - QT_big : j);
      const int64_t bh = __builtin_amdgcn_readfirstlane(pair % BH);
      const int jid = __builtin_amdgcn_readfirstlane(pair / BH);
      attn_tile<D, 2>(smem, q, jobs, jid, bh, int64_t(qt) * Tile<D, 2>::BM, Nq, scale_log2);
    } else {
      const int pa = 2 * pp, pb = has_b ? 2 * pp + 1 : 2 * pp;
      const int64_t bh_a = __builtin_amdgcn_readfirstlane(pa % BH);
      const int jid_a = __builtin_amdgcn_readfirstlane(pa / BH);
      const int64_t bh_b = __builtin_amdgcn_readfirstlane(pb % BH);
      const int jid_b = __builtin_amdgcn_readfirstlane(pb / BH);
      const int64_t tail0 = int64_t(QT_big) * Tile<D, 2>::BM;
      attn_tile<D, 1, false, 0, true>(smem, q, jobs, jid_a, bh_a, tail0, Nq, scale_log2, 0, -1,
                                      jid_b, bh_b, has_b ? tail0 : int64_t(Nq));
    }
    return;
  } else if constexpr (!SPLIT) {
    int pair;
    int64_t row0;
    bool big;
    if (stage_a >= 0) {
      big = pid < n_big;
      const int lin = __builtin_amdgcn_readfirstlane(
          int(big ? xcd_remap(pid, n_big) : xcd_remap(pid - n_big, n_small)));
      const StagedTile st = staged_tile(lin, big, QT_big, QT_small, QT_small_b, stage_a);
      pair = __builtin_amdgcn_readfirstlane(int(st.pair));
      row0 = __builtin_amdgcn_readfirstlane(int(st.row0));
    } else {
      // The tiles of one (head, block) are consecutive, its 256-row tiles right
      // after its 512-row ones, so they read the block's K/V from the same L2.
      const int per_pair = QT_big + QT_small;
      const int lin = __builtin_amdgcn_readfirstlane(int(xcd_remap(pid, n_big + n_small)));
      const int j = __builtin_amdgcn_readfirstlane(lin % per_pair);
      pair = __builtin_amdgcn_readfirstlane(lin / per_pair);
      big = j < QT_big;
      row0 = big ? int64_t(j) * Tile<D, 2>::BM
                 : int64_t(QT_big) * Tile<D, 2>::BM + int64_t(j - QT_big) * Tile<D, 1>::BM;
    }
    const int64_t bh = __builtin_amdgcn_readfirstlane(pair % BH);
    const int jid = __builtin_amdgcn_readfirstlane(pair / BH);
    if (big)
      attn_tile<D, 2>(smem, q, jobs, jid, bh, row0, Nq, scale_log2);
    else
      attn_tile<D, 1>(smem, q, jobs, jid, bh, row0, Nq, scale_log2);
    return;
  } else {
    SplitShared* sh = split_shared();
    int64_t lin, r = -1, second_end = 0;
    int kt0 = 0, kt1 = -1;
    if (pid < n_big) {
      lin = xcd_remap(pid, n_big);
    } else {
      // Split unit u: its range [x, hi) is at most a tile long; the first
      // segment runs to the end of the tile it starts in (or to hi), the second
      // from the next tile boundary to hi.
      const int64_t u = pid - n_big;
      const int T = sa.plan.T;
      const int64_t x = split_lo(sa.plan, u), hi = split_lo(sa.plan, u + 1);
      const int64_t edge = (x / T + 1) * T;
      r = x / T;
      kt0 = int(x - r * T);
      kt1 = int((hi < edge ? hi : edge) - r * T);
      if (hi > edge) second_end = hi - edge;
      lin = n_big + r;
      if (kt0 == 0 && kt1 == T) r = -1;  // a unit range that is exactly one tile
      if (threadIdx.x == 0) {
        sh->plan = sa.plan;
        sh->pieces = sa.pieces;
        sh->count = sa.count;
        sh->unit = u;
      }
    }
    if (threadIdx.x == 0) sh->r = r;
    __syncthreads();  // the split state is written before any wave reads it
    {
      const int qt = __builtin_amdgcn_readfirstlane(int(lin % QT_big));
      const int rest = __builtin_amdgcn_readfirstlane(int(lin / QT_big));
      const int64_t bh = __builtin_amdgcn_readfirstlane(rest % BH);
      const int jid = __builtin_amdgcn_readfirstlane(rest / BH);
      attn_tile<D, 2, true>(smem, q, jobs, jid, bh, int64_t(qt) * Tile<D, 2>::BM, Nq, scale_log2,
                            kt0, kt1);
    }
    if (second_end == 0) return;
    // The unit's second segment: key tiles [0, second_end) of the next tile.
    // Its parameters are recomputed from the block index, not kept live through
    // the first segment's main loop.
    __syncthreads();  // the first segment's LDS reads are done
    {
      const int64_t u2 = int64_t(blockIdx.x) - n_big;
      const int T = sa.plan.T;
      const int64_t x = split_lo(sa.plan, u2), hi = split_lo(sa.plan, u2 + 1);
      const int64_t r2 = x / T + 1;
      const int kt1b = int(hi - r2 * T);
      const int64_t lin2 = n_big + r2;
      if (threadIdx.x == 0) sh->r = kt1b == T ? -1 : r2;
      __syncthreads();
      const int qt = __builtin_amdgcn_readfirstlane(int(lin2 % QT_big));
      const int rest = __builtin_amdgcn_readfirstlane(int(lin2 / QT_big));
      const int64_t bh = __builtin_amdgcn_readfirstlane(rest % BH);
      const int jid = __builtin_amdgcn_readfirstlane(rest / BH);
      attn_tile<D, 2, true, 1>(smem, q, jobs, jid, bh, int64_t(qt) * Tile<D, 2>::BM, Nq,
                               scale_log2, 0, kt1b);
    }
  }
}

// Launch layout: 512-row and 256-row tiles per (head, block), and the key
// split of the remainder (sa.plan.units == 0: none; the scratch pointers are
// filled in at launch).
struct LaunchPlan {
  TileSplit split;
  int64_t n_big;
  int64_t n_small;   // 256-row workgroups (DUAL: one per two pairs)
  SplitArgs sa;
  bool dual;         // tails of two (head, block) pairs per 256-row workgroup
  int64_t pairs;     // (head, block) pairs of the launch
  int stage_a = -1;  // staged layout: pairs with split.big 512-row tiles (< 0: none)
  int small_b = 0;   // staged layout: 256-row tiles of the other pairs
};

// Extra cost of one split segment (restarting the K/V pipeline, storing the
// piece, reloading the pieces it combines), in key-tile iterations.
constexpr int kSegmentCost = 4;
// Measured on one MI355X (4725 keys per block, 40 heads, D = 128): a split
// unit's key-tile iteration takes 1.1-1.2x a whole tile's when the block's K
// and V sit in the memory-side cache and ~1.85x when they come from HBM (a
// whole tile shares every K/V tile with the other query tiles of its (head,
// block) running beside it on the XCD; a unit streams its own key range), and
// the whole-tile rounds before the units end over a spread of ~0.07 tile
// times per round (a unit starts when its compute unit frees up).  The
// planner takes the HBM figure: a single call on 4725 x 4725 x 40 heads (one
// round and a 0.56 remainder) measured 11% slower split, three blocks (four
// rounds and a 0.69 remainder) 2% slower; launches with fewer tiles than
// compute units are split (the units' parallelism outweighs the lost sharing).
constexpr double kSplitIterCost = 1.85;
constexpr double kRoundSpread = 0.07;
// Arrival counters of a launch (one per remainder tile) in the scratch.
constexpr size_t kCounterBytes = kSplitMaxCounters * sizeof(int);

// Key split of the last round of n 512-row tiles (T key tiles each), if its
// estimate finishes 3% before t_tiles; units == 0: none.
SplitPlan choose_key_split(int64_t n, int cus, int T, double t_tiles) {
  const SplitPlan none{};
  const int64_t rem = n % cus;
  if (T < 2 || rem == 0) return none;  // unequal key lengths (T = 0), one key tile, whole rounds
  // Early reject by the split's best case (the most units, hence the shortest
  // ranges) before the planner checks every tile's pieces.
  const int per_tile = std::max(4, std::min(kSplitMaxUnitsPerTile, T / kSplitMinIters));
  const int64_t most_units = std::min<int64_t>(std::min(cus, kSplitMaxUnits), rem * std::min(per_tile, T));
  if (most_units <= rem) return none;
  const double best = double(n / cus) * (1.0 + kRoundSpread) +
                      kSplitIterCost * double((rem * T + most_units - 1) / most_units +
                                              2 * kSegmentCost) / double(T);
  if (best >= 0.97 * t_tiles) return none;
  double t_units = 0.0;
  const SplitPlan sk = plan_key_split(n, cus, T, kSegmentCost, &t_units);
  const double rounds = double(n / cus);
  const double t_split = rounds * (1.0 + kRoundSpread) + kSplitIterCost * (t_units - rounds);
  return sk.units > 0 && t_split < 0.97 * t_tiles ? sk : none;
}

// Layout of a launch of `per` (head, block) pairs of Nq query rows, T key
// tiles each (T = 0: unequal key lengths), on `cus` compute units: dual tails
// where they finish first; otherwise the key split where it beats the
// per-pair layouts (measured: it does on launches of few tiles, where the
// staged layout's estimate can be lower); otherwise the staged layout where
// its estimate is lower than the per-pair layouts'.
LaunchPlan plan_launch(int64_t Nq, int64_t per, int cus, int T) {
  LaunchPlan lp{};
  lp.pairs = per;
  lp.split = choose_tile_split(Nq, per, cus);
  lp.n_big = int64_t(lp.split.big) * per;
  lp.n_small = int64_t(lp.split.small) * per;
  const double t_tiles = estimated_makespan(lp.n_big, lp.n_small, cus, kSmallTileCost);
  // All 512-row tiles first, sized to fill whole rounds, then all 256-row ones.
  double t_staged = 0.0;
  const StagedLayout sl = plan_staged(Nq, per, cus, kSmallTileCost, &t_staged);
  const bool staged = sl.stage_a >= 0 && t_staged < t_tiles - 1e-9;
  // Tails of at most 128 rows, two per 256-row workgroup (the pairs must have
  // one key length), when that finishes earlier than the layouts above.
  const int whole = int(Nq / 512);
  const int64_t tail = Nq - int64_t(whole) * 512;
  if (T > 0 && tail > 0 && tail <= 128 && per >= 2) {
    const int64_t n_dual = (per + 1) / 2;
    const double t_dual = estimated_makespan(int64_t(whole) * per, n_dual, cus, kDualTileCost);
    if (t_dual < t_tiles - 1e-9 && (!staged || t_dual < t_staged - 1e-9)) {
      lp.split = TileSplit{whole, 1};
      lp.n_big = int64_t(whole) * per;
      lp.n_small = n_dual;
      lp.dual = true;
      return lp;  // no key split with dual tails
    }
  }
  const int all_big = int((Nq + 511) / 512);
  const int64_t n = int64_t(all_big) * per;
  const SplitPlan sk = choose_key_split(n, cus, T, t_tiles);
  if (sk.units > 0) {
    lp.split = TileSplit{all_big, 0};
    lp.n_big = n - sk.rem;
    lp.n_small = 0;
    lp.sa.plan = sk;
  } else if (staged) {
    lp.split = TileSplit{sl.nb, sl.ns_a};
    lp.n_big = sl.n_big;
    lp.n_small = sl.n_small;
    lp.stage_a = sl.stage_a;
    lp.small_b = sl.ns_b;
  }
  return lp;
}

// Scratch of the key split, one per device: arrival counters (zeroed when
// allocated; every launch leaves them zero) and piece slots for the most
// units any launch uses, at D = 128 (the larger pieces).  Allocated once, on
// the first split launch on the device, and never moved or freed, so a launch
// captured in a graph keeps a valid address for every replay.  Launches that
// use it are ordered by an event when they come from different streams.  A
// launch under stream capture uses it as it is, without waiting or recording
// (the caller orders replays, e.g. on the stream the other calls use); one
// captured before the scratch exists runs without the split.
constexpr size_t kScratchBytes = kCounterBytes + size_t(2) * kSplitMaxUnits * Tile<128>::PIECE;
struct SplitScratch {
  std::mutex mu;
  char* base = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  hipStream_t last = nullptr;
  bool used = false;
};
SplitScratch g_scratch[64];

template <int D>
hipError_t launch_d(const AttnProblem& pr, const void* q, const AttnJobs& jobs,
                    const LaunchPlan& lp, hipStream_t stream) {
  const int64_t n_split = lp.sa.plan.units;
  const int64_t n = lp.n_big + lp.n_small + n_split;
  const int pairs = int(lp.pairs);
  if (n_split == 0 && !lp.dual)
    attn_fwd_bf16_kernel<D, false><<<dim3(unsigned(n)), Tile<D>::kThreads, 0, stream>>>(
        static_cast<const __bf16*>(q), jobs, int(pr.Nq), pr.BH, int(lp.n_big), lp.split.big,
        int(lp.n_small), lp.split.small, lp.sa, pr.scale * kLog2e, pairs, lp.stage_a, lp.small_b);
  else if (n_split == 0)
    attn_fwd_bf16_kernel<D, false, true><<<dim3(unsigned(n)), Tile<D>::kThreads, 0, stream>>>(
        static_cast<const __bf16*>(q), jobs, int(pr.Nq), pr.BH, int(lp.n_big), lp.split.big,
        int(lp.n_small), lp.split.small, lp.sa, pr.scale * kLog2e, pairs, lp.stage_a, lp.small_b);
  else
    attn_fwd_bf16_kernel<D, true><<<dim3(unsigned(n)), Tile<D>::kThreads, 0, stream>>>(
        static_cast<const __bf16*>(q), jobs, int(pr.Nq), pr.BH, int(lp.n_big), lp.split.big,
        int(lp.n_small), lp.split.small, lp.sa, pr.scale * kLog2e, pairs, lp.stage_a, lp.small_b);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                        LaunchPlan& lp, int cus, int dev, hipStream_t stream) {
  if (lp.sa.plan.units == 0) return launch_d<D>(pr, q, jobs, lp, stream);
  SplitScratch& w = g_scratch[dev];
  std::lock_guard<std::mutex> lock(w.mu);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return e;
  const bool capturing = cap != hipStreamCaptureStatusNone;
  static_assert(sizeof(int) * kSplitMaxCounters == kCounterBytes, "counter region");
  if (lp.sa.plan.units > kSplitMaxUnits || lp.sa.plan.rem > kSplitMaxCounters)
    return hipErrorInvalidValue;  // the planner keeps to both
  if (!w.base) {
    if (capturing)  // no allocation under capture: the layout without the split
      return launch_d<D>(pr, q, jobs, plan_launch(pr.Nq, int64_t(pr.BH) * n_jobs, cus, 0), stream);
    if ((e = hipMalloc(&w.base, kScratchBytes)) != hipSuccess) {
      w.base = nullptr;
      return e;
    }
    if ((e = hipMemsetAsync(w.base, 0, kCounterBytes, stream)) != hipSuccess) return e;
    w.bytes = kScratchBytes;
  }
  if (!capturing) {
    if (!w.done && (e = hipEventCreateWithFlags(&w.done, hipEventDisableTiming)) != hipSuccess)
      return e;
    if (w.used && w.last != stream && (e = hipStreamWaitEvent(stream, w.done, 0)) != hipSuccess)
      return e;
  }
  lp.sa.count = reinterpret_cast<int*>(w.base);
  lp.sa.pieces = w.base + kCounterBytes;
  if ((e = launch_d<D>(pr, q, jobs, lp, stream)) != hipSuccess) return e;
  if (!capturing) {
    if ((e = hipEventRecord(w.done, stream)) != hipSuccess) return e;
    w.last = stream;
    w.used = true;
  }
  return hipSuccess;
}

}  // namespace

hipError_t attn_bf16_layout(const AttnProblem& pr, int n_jobs, int64_t nk, AttnLayout* out) {
  int cus = 0;
  const hipError_t e = compute_units(&cus);
  if (e != hipSuccess) return e;
  const int BN = 4096 / pr.D;
  const int T = nk > 0 ? int((nk + BN - 1) / BN) : 0;
  const LaunchPlan lp = plan_launch(pr.Nq, int64_t(pr.BH) * n_jobs, cus, T);
  const int units = lp.sa.plan.units;
  out->big = lp.split.big;
  out->small = lp.split.small;
  out->dual = lp.dual ? 1 : 0;
  out->stage_a = lp.stage_a;
  out->small_b = lp.small_b;
  out->units = units;
  out->rem = units > 0 ? lp.sa.plan.rem : 0;
  int most = 0;
  for (int64_t r = 0; r < out->rem; ++r) most = std::max(most, split_pieces(lp.sa.plan, r));
  out->max_pieces = most;
  out->workgroups = lp.n_big + lp.n_small + units;
  out->cus = cus;
  const int piece = pr.D == 128 ? Tile<128>::PIECE : Tile<64>::PIECE;
  out->scratch = units > 0 ? int64_t(kCounterBytes) + int64_t(2) * units * piece : 0;
  out->scratch_allocated = units > 0 ? int64_t(kScratchBytes) : 0;
  return hipSuccess;
}

hipError_t launch_attn_bf16(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                            hipStream_t stream) {
  int cus = 0, dev = 0;
  const hipError_t e = compute_units(&cus, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  // The key split needs one key length for every block of the launch.
  int T = 0;
  const int BN = 4096 / pr.D;
  bool same = n_jobs > 0;
  for (int j = 1; j < n_jobs; ++j) same &= jobs.job[j].nk == jobs.job[0].nk;
  if (same) T = int((jobs.job[0].nk + BN - 1) / BN);
  LaunchPlan lp = plan_launch(pr.Nq, int64_t(pr.BH) * n_jobs, cus, T);
  return pr.D == 128 ? launch_split<128>(pr, q, jobs, n_jobs, lp, cus, dev, stream)
                     : launch_split<64>(pr, q, jobs, n_jobs, lp, cus, dev, stream);
}

}  // namespace dita
