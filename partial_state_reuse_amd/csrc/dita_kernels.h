// Internal interface between the C ABI (api.hip) and the device kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dita {

constexpr int kMaxParts = 64;

// One fresh (query partition, KV partition) block of a grouped attention launch.
struct AttnJob {
  const void* k;   // [B, H, nk, D]
  const void* v;   // [B, H, nk, D]
  void* o;         // [B, H, Nq, D]
  float* lse;      // [B, H, Nq]
  int64_t nk;
};

struct AttnJobs {
  AttnJob job[kMaxParts];
};

struct AttnProblem {
  int BH;          // B * H
  int D;           // 64 or 128
  int64_t Nq;
  float scale;     // softmax scale (> 0)
};

// bf16 Q/K/V/O, MFMA with fp32 accumulation.  Launches grid.z = n_jobs.
hipError_t launch_attn_bf16(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                            hipStream_t stream);
// Work layout launch_attn_bf16 uses on the current device for n_jobs blocks of
// nk keys each (nk <= 0: blocks of unequal lengths).
struct AttnLayout {
  int big, small;      // 512-row and 256-row tiles per (head, block)
  int dual;            // 1: each 256-row workgroup takes the tails of two pairs
  int64_t workgroups;
  int units, rem, max_pieces;
  int cus;
  int64_t scratch;     // bytes of the key-split scratch this launch uses
  int64_t scratch_allocated;  // bytes the library holds for it per device
  int stage_a;         // staged layout: pairs with `big` and `small` tiles (< 0: none)
  int small_b;         // staged layout: 256-row tiles of the other pairs (big - 1 512-row)
};
hipError_t attn_bf16_layout(const AttnProblem& pr, int n_jobs, int64_t nk, AttnLayout* out);
// fp32 throughout.
hipError_t launch_attn_f32(const AttnProblem& pr, const void* q, const AttnJobs& jobs, int n_jobs,
                           hipStream_t stream);

// Sources of a merge.  scale[p] == nullptr: o[p] is a state's output in the
// merge dtype; otherwise (bf16 merges only) o[p] holds the int8 codes of a
// compact state and scale[p] its per-row scales.
struct MergeSrc {
  const void* o[kMaxParts];
  const float* lse[kMaxParts];
  const float* scale[kMaxParts];
};

// Optional second output of a merge: the merge of sources [first, end) alone
// (a group state composed in the same pass), written to (o, lse).  o may be
// the output of source `first` (in place).  end <= first: none.
struct MergeGroup {
  int first, end;
  void* o;
  float* lse;
};

// P-way LSE merge over `rows` = B*H*Nq rows of D elements.  dtype: 0 fp32, 1 bf16.
hipError_t launch_merge(int dtype, int D, int64_t rows, int P, const MergeSrc& src, void* o,
                        float* lse, hipStream_t stream, const MergeGroup& group = MergeGroup{});

struct LseList {
  const float* lse[kMaxParts];
};

// w[p] = mean over `rows` rows of exp(LSE_p - LSE) (fp64), one workgroup per partition.
hipError_t launch_contrib(int P, const LseList& src, const float* lse, int64_t rows, double* w,
                          hipStream_t stream);

// out[0] = sum (new - prev)^2, out[1] = sum prev^2, out[2] = sqrt(out[0] / out[1]) over the
// O elements (fp64, summation order fixed by o_bytes); roll != 0 also copies the new state
// (O and LSE) over prev.  `partials` holds 2 * change_groups(o_bytes) doubles of scratch.
constexpr int kChangeMaxGroups = 1024;
int change_groups(size_t o_bytes);
hipError_t launch_change(int dtype, const void* o_new, void* o_prev, size_t o_bytes,
                         const float* lse_new, float* lse_prev, size_t lse_bytes, int roll,
                         double* partials, double* out, hipStream_t stream);

// Compact encoding of a bf16 state of `rows` rows of D: int8 codes [rows, D],
// fp32 scale [rows], and the LSE copied to lse_out.
hipError_t launch_compact_encode(int D, const void* o, const float* lse, int8_t* codes,
                                 float* scale, float* lse_out, int64_t rows, hipStream_t stream);

// Copy of one attention state (O bytes and LSE bytes, each a multiple of 4 bytes).
hipError_t launch_copy_state(const void* src_o, const float* src_lse, void* dst_o, float* dst_lse,
                             size_t o_bytes, size_t lse_bytes, hipStream_t stream);

}  // namespace dita
