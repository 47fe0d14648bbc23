// C ABI: argument validation, the state-cache handle, and rank-step dispatch.
//
// Every entry point validates all of its arguments before it makes any HIP
// call, so a rejected call launches nothing and changes nothing.  Launches are
// asynchronous on the caller's stream; the library never synchronises.
//
// The cache handle keeps host metadata only: per partition its validity, the
// step that wrote its state, its group (composed partitions share the state
// in the group's first slot; the DiTango page, State-Centric Parallel Runtime >
// Dynamic Group Compose), the physical slot holding its state (fixed, or taken
// from a pool) and, for a state moved to the host, the caller's buffers.  A
// step widens the caller's mask to whole groups, takes physical slots for what
// it computes or brings back, launches one grouped attention kernel writing
// straight into the slots, and merges one state per group; with a side stream
// it copies host-resident states back, and may pre-merge the reused ones,
// beside the attention (Pipeline Orchestration on the same page).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/dita.h"
#include "dita_kernels.h"
#include "planner.h"

struct dita_state_cache {
  dita_shape shape;
  int P;
  char* base;
  size_t bytes;
  size_t o_bytes;      // bytes of one slot's O
  size_t lse_offset;   // offset of LSE inside a slot
  size_t slot_stride;  // bytes per slot
  uint8_t valid[DITA_MAX_PARTITIONS];
  int64_t stamp[DITA_MAX_PARTITIONS];
  int16_t group[DITA_MAX_PARTITIONS];  // leader (first partition) of p's group
  hipEvent_t ev_fork;                  // stream -> side stream, created on first use
  hipEvent_t ev_join;                  // side stream -> stream
  int S;                               // physical (full) slots in the buffer
  bool pool;                           // slots assigned on demand; else partition p owns slot p
  int16_t phys[DITA_MAX_PARTITIONS];   // physical slot holding p's own state, -1 if none
  // Compact slots (int8 codes + per-row scale + LSE), after the S full slots;
  // a state is held in a full slot, a compact slot or host memory, never two.
  int C;
  size_t c_base;                       // offset of compact slot 0
  size_t c_scale_off, c_lse_off;       // offsets of the scales and the LSE inside one
  size_t c_stride;                     // bytes per compact slot
  int16_t cphys[DITA_MAX_PARTITIONS];  // compact slot holding p's state, -1 if none
  uint8_t on_host[DITA_MAX_PARTITIONS];  // p's state lives in caller host memory
  void* host_o[DITA_MAX_PARTITIONS];
  float* host_lse[DITA_MAX_PARTITIONS];
  // Pooled caches only: the event recorded after the last device work that
  // touched each physical slot, and the stream it was recorded on.  Events are
  // shared by the slots one call touched (reference counted) and created on
  // first use.
  int16_t slot_ev[DITA_MAX_PARTITIONS];   // index into ev, -1 if no work is tracked
  hipEvent_t ev[DITA_MAX_PARTITIONS + 1];
  void* ev_stream[DITA_MAX_PARTITIONS + 1];
  int16_t ev_refs[DITA_MAX_PARTITIONS + 1];
};

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxRows = int64_t(1) << 30;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return DITA_OK;
  g_last_hip_error = int(e);
  return DITA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_size(int dtype) { return dtype == DITA_BF16 ? 2 : 4; }

int check_shape(const dita_shape* s) {
  if (!s) return DITA_ERR_ARG;
  if (s->dtype != DITA_F32 && s->dtype != DITA_BF16) return DITA_ERR_DTYPE;
  if (s->B < 1 || s->H < 1 || int64_t(s->B) * s->H > 65535) return DITA_ERR_SHAPE;
  if (s->D != 64 && s->D != 128) return DITA_ERR_SHAPE;
  if (s->Nq < 1 || s->Nq > kMaxRows) return DITA_ERR_SHAPE;
  if (std::isnan(s->scale) || std::isinf(s->scale)) return DITA_ERR_ARG;
  return DITA_OK;
}

int check_dev(const void* p) {
  if (!p) return DITA_ERR_ARG;
  return aligned16(p) ? DITA_OK : DITA_ERR_ALIGN;
}

float eff_scale(const dita_shape& s) { return s.scale > 0.0f ? s.scale : 1.0f / std::sqrt(float(s.D)); }

size_t state_o_bytes(const dita_shape& s) {
  return size_t(s.B) * size_t(s.H) * size_t(s.Nq) * size_t(s.D) * elem_size(s.dtype);
}
size_t state_lse_bytes(const dita_shape& s) { return size_t(s.B) * size_t(s.H) * size_t(s.Nq) * 4; }

// A K or V head slice must stay below 2^31 bytes: the attention kernel
// addresses it through a buffer resource with a 32-bit record count.
bool nk_ok(const dita_shape& s, int64_t nk) {
  return nk >= 1 && nk <= kMaxRows && nk * int64_t(s.D) * int64_t(elem_size(s.dtype)) < (int64_t(1) << 31);
}

dita::AttnProblem problem(const dita_shape& s) {
  dita::AttnProblem pr;
  pr.BH = s.B * s.H;
  pr.D = s.D;
  pr.Nq = s.Nq;
  pr.scale = eff_scale(s);
  return pr;
}

hipError_t launch_attn(const dita_shape& s, const void* q, const dita::AttnJobs& jobs, int n,
                       hipStream_t st) {
  const dita::AttnProblem pr = problem(s);
  return s.dtype == DITA_BF16 ? dita::launch_attn_bf16(pr, q, jobs, n, st)
                              : dita::launch_attn_f32(pr, q, jobs, n, st);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_slot(const dita_state_cache* c, int p) {
  if (!c) return DITA_ERR_ARG;
  if (p < 0 || p >= c->P) return DITA_ERR_ARG;
  return DITA_OK;
}

void* phys_o(const dita_state_cache* c, int k) { return c->base + size_t(k) * c->slot_stride; }
float* phys_lse(const dita_state_cache* c, int k) {
  return reinterpret_cast<float*>(c->base + size_t(k) * c->slot_stride + c->lse_offset);
}
// Device state of partition p (its physical slot must be assigned).
void* slot_o(const dita_state_cache* c, int p) { return phys_o(c, c->phys[p]); }
float* slot_lse(const dita_state_cache* c, int p) { return phys_lse(c, c->phys[p]); }

char* cslot(const dita_state_cache* c, int j) { return c->base + c->c_base + size_t(j) * c->c_stride; }
int8_t* cslot_codes(const dita_state_cache* c, int j) { return reinterpret_cast<int8_t*>(cslot(c, j)); }
float* cslot_scale(const dita_state_cache* c, int j) {
  return reinterpret_cast<float*>(cslot(c, j) + c->c_scale_off);
}
float* cslot_lse(const dita_state_cache* c, int j) {
  return reinterpret_cast<float*>(cslot(c, j) + c->c_lse_off);
}

// A state that is valid, leads its group and sits in a full device slot.
bool resident(const dita_state_cache* c, int p) {
  return c->valid[p] && c->group[p] == p && c->phys[p] >= 0 && !c->on_host[p];
}
// ... or in a full or compact device slot.
bool on_device(const dita_state_cache* c, int p) {
  return c->valid[p] && c->group[p] == p && !c->on_host[p] && (c->phys[p] >= 0 || c->cphys[p] >= 0);
}

// The device LSE of a leader on the device.
const float* state_lse(const dita_state_cache* c, int p) {
  return c->cphys[p] >= 0 ? cslot_lse(c, c->cphys[p]) : slot_lse(c, p);
}

// Append leader p's device state (either format) to a merge's sources.
void add_source(const dita_state_cache* c, dita::MergeSrc& src, int& n, int p) {
  if (c->cphys[p] >= 0) {
    const int j = c->cphys[p];
    src.o[n] = cslot_codes(c, j);
    src.lse[n] = cslot_lse(c, j);
    src.scale[n] = cslot_scale(c, j);
  } else {
    src.o[n] = slot_o(c, p);
    src.lse[n] = slot_lse(c, p);
    src.scale[n] = nullptr;
  }
  ++n;
}

// Lowest physical slot that no partition holds and `taken` does not mark; marks it.
int take_free(const dita_state_cache* c, uint64_t* taken) {
  uint64_t used = *taken;
  for (int p = 0; p < c->P; ++p)
    if (c->phys[p] >= 0) used |= uint64_t(1) << c->phys[p];
  for (int k = 0; k < c->S; ++k)
    if (!((used >> k) & 1)) {
      *taken |= uint64_t(1) << k;
      return k;
    }
  return -1;
}

// Lowest compact slot that no partition holds; -1 if none.
int take_free_compact(const dita_state_cache* c) {
  uint64_t used = 0;
  for (int p = 0; p < c->P; ++p)
    if (c->cphys[p] >= 0) used |= uint64_t(1) << c->cphys[p];
  for (int j = 0; j < c->C; ++j)
    if (!((used >> j) & 1)) return j;
  return -1;
}

// In a pooled cache a partition without a state of its own holds no slot.
void release(dita_state_cache* c, int p) {
  if (c->pool) c->phys[p] = -1;
  c->cphys[p] = -1;
}

void forget_host(dita_state_cache* c, int p) {
  c->on_host[p] = 0;
  c->host_o[p] = nullptr;
  c->host_lse[p] = nullptr;
}

// Last partition of the group led by `first`.
int group_last(const dita_state_cache* c, int first) {
  int last = first;
  while (last + 1 < c->P && c->group[last + 1] == first) ++last;
  return last;
}

void reset_slot(dita_state_cache* c, int p) {
  c->valid[p] = 0;
  c->stamp[p] = -1;
  c->group[p] = int16_t(p);
  forget_host(c, p);
  release(c, p);
}

// The mask a step applies: a group of two or more is reused only when every
// member is marked reuse.  Returns DITA_ERR_ARG for mask values other than
// 0/1 and DITA_ERR_STATE for reuse of an invalid slot.
int effective_mask(const dita_state_cache* c, const uint8_t* reuse, uint8_t* out) {
  for (int p = 0; p < c->P; ++p) {
    if (reuse[p] > 1) return DITA_ERR_ARG;
    if (reuse[p] && !c->valid[p]) return DITA_ERR_STATE;
  }
  for (int p = 0; p < c->P;) {
    const int last = group_last(c, p);
    uint8_t all = 1;
    for (int i = p; i <= last; ++i) all &= reuse[i];
    for (int i = p; i <= last; ++i) out[i] = last > p ? all : reuse[i];
    p = last + 1;
  }
  return DITA_OK;
}

// Stream order of pooled slots.  A pooled cache hands a physical slot from one
// partition to another, so work the caller enqueued on one stream for the old
// owner (a copy to the host, a merge reading it) may still be pending when a
// call on another stream writes the new owner's state there.  Every call that
// enqueues device work on pooled slots therefore first makes its stream wait
// for the last recorded work on each slot it touches (when that was recorded
// on a different stream), and afterwards records one event on its stream for
// all of them: device work on one pooled slot runs in call order, whatever the
// streams.  Unpooled caches skip this (partition p owns slot p; ordering work
// on a partition's slot is the caller's, as for any device buffer).
int slots_wait(dita_state_cache* c, hipStream_t s, uint64_t slots) {
  if (!c->pool) return DITA_OK;
  uint64_t waited = 0;
  for (int k = 0; k < c->S + c->C; ++k) {
    if (!((slots >> k) & 1)) continue;
    const int e = c->slot_ev[k];
    if (e < 0 || ((waited >> e) & 1) || c->ev_stream[e] == static_cast<void*>(s)) continue;
    const int st = hip_status(hipStreamWaitEvent(s, c->ev[e], 0));
    if (st) return st;
    waited |= uint64_t(1) << e;
  }
  return DITA_OK;
}

int slots_mark(dita_state_cache* c, hipStream_t s, uint64_t slots) {
  if (!c->pool || !slots) return DITA_OK;
  // A free event: at most S + C <= 64 are referenced by slots, and there are 65.
  int e = 0;
  while (c->ev_refs[e] > 0) ++e;
  int st;
  if (!c->ev[e] && (st = hip_status(hipEventCreateWithFlags(&c->ev[e], hipEventDisableTiming))))
    return st;
  if ((st = hip_status(hipEventRecord(c->ev[e], s)))) return st;
  c->ev_stream[e] = static_cast<void*>(s);
  for (int k = 0; k < c->S + c->C; ++k) {
    if (!((slots >> k) & 1)) continue;
    if (c->slot_ev[k] >= 0) --c->ev_refs[c->slot_ev[k]];
    c->slot_ev[k] = int16_t(e);
    ++c->ev_refs[e];
  }
  return DITA_OK;
}

uint64_t slot_bit(int k) { return k >= 0 ? uint64_t(1) << k : 0; }
// Ordering bit of compact slot j (after the full slots).
uint64_t cslot_bit(const dita_state_cache* c, int j) { return j >= 0 ? uint64_t(1) << (c->S + j) : 0; }
// Ordering bit of the slot holding leader p's device state (either format).
uint64_t state_bit(const dita_state_cache* c, int p) {
  return c->cphys[p] >= 0 ? cslot_bit(c, c->cphys[p]) : slot_bit(c->phys[p]);
}

// Where composing first..last writes the group state: the full slot of
// `first` if it has one, else that of the first leader in the range with one
// (the merge then runs in place, that state being source 0), else a free full
// slot (marked in *taken; out of place).  Returns the slot, -1 if none is
// free; *src0 is the leader read as source 0 in place, or -1.
int compose_output(const dita_state_cache* c, int first, int last, uint64_t* taken, int* src0) {
  *src0 = -1;
  if (c->phys[first] >= 0) {
    *src0 = first;
    return c->phys[first];
  }
  for (int p = first + 1; p <= last; ++p)
    if (c->group[p] == p && c->phys[p] >= 0) {
      *src0 = p;
      return c->phys[p];
    }
  return take_free(c, taken);
}

// Number of group leaders in first..last.
int leaders_in(const dita_state_cache* c, int first, int last) {
  int n = 0;
  for (int p = first; p <= last; ++p) n += c->group[p] == p ? 1 : 0;
  return n;
}

// Compose partitions first..last (validated by the caller: all valid, every
// leader on the device, no group straddling the range, and an output slot from
// compose_output when two or more leaders take part) into one group state held
// by `first`.
// Cache records of a composition of first..last once its merge is enqueued
// (out_k: the slot it wrote; -1: one leader, nothing merged): the members'
// slots go back to the pool, `first` leads the group with the oldest stamp.
void finish_compose(dita_state_cache* c, int first, int last, int out_k) {
  int64_t oldest = c->stamp[first];
  for (int p = first; p <= last; ++p)
    if (c->group[p] == p && c->stamp[p] < oldest) oldest = c->stamp[p];
  if (out_k >= 0) {
    for (int p = first; p <= last; ++p) release(c, p);
    c->phys[first] = int16_t(out_k);
  } else {
    for (int p = first + 1; p <= last; ++p) release(c, p);
  }
  for (int p = first; p <= last; ++p) {
    c->group[p] = int16_t(first);
    c->valid[p] = 1;
    c->stamp[p] = oldest;
  }
}

int compose_range(dita_state_cache* c, int first, int last, int out_k, int src0, hipStream_t stream,
                  int* launched) {
  // `first` leads its group: no group straddles the range and first is in it.
  dita::MergeSrc src{};
  int n = 0;
  uint64_t touched = slot_bit(out_k);
  if (src0 >= 0) add_source(c, src, n, src0);
  for (int p = first; p <= last; ++p)
    if (c->group[p] == p) {
      if (p != src0) add_source(c, src, n, p);
      touched |= state_bit(c, p);
    }
  if (n > 1) {
    // In place when src0 >= 0: the output is source 0; each lane reads its
    // elements of every source before it writes them.
    const dita_shape& s = c->shape;
    const int64_t rows = int64_t(s.B) * s.H * s.Nq;
    int st = slots_wait(c, stream, touched);
    if (st) return st;
    st = hip_status(
        dita::launch_merge(s.dtype, s.D, rows, n, src, phys_o(c, out_k), phys_lse(c, out_k), stream));
    if (st) return st;
    // The members' slots go back to the pool below: their next owner waits for this merge.
    if ((st = slots_mark(c, stream, touched))) return st;
  }
  finish_compose(c, first, last, n > 1 ? out_k : -1);
  if (launched) *launched = n > 1 ? 1 : 0;
  return DITA_OK;
}

// The runs dita_state_cache_compose_runs composes for a reuse mask: maximal
// runs of reused partitions, shrunk to the groups that lie inside them, that
// hold two or more groups.  DITA_ERR_ARG for mask values other than 0/1,
// DITA_ERR_STATE for reuse of an invalid state or of a group leader that is
// not on the device (fetch it first).
int plan_runs(const dita_state_cache* c, const uint8_t* reuse, int* first, int* last, int* n_out) {
  for (int p = 0; p < c->P; ++p) {
    if (reuse[p] > 1) return DITA_ERR_ARG;
    if (reuse[p] && !c->valid[p]) return DITA_ERR_STATE;
  }
  int n = 0;
  for (int p = 0; p < c->P;) {
    if (!reuse[p]) {
      ++p;
      continue;
    }
    int a = p, b = p;
    while (b + 1 < c->P && reuse[b + 1]) ++b;
    p = b + 1;
    // Groups that reach outside the run will be recomputed whole: leave them out.
    if (c->group[a] < a) a = group_last(c, c->group[a]) + 1;
    if (b >= a && group_last(c, c->group[b]) > b) b = c->group[b] - 1;
    if (a < b && !(c->group[a] == a && group_last(c, a) == b)) {
      first[n] = a;
      last[n] = b;
      ++n;
    }
  }
  for (int i = 0; i < n; ++i)
    for (int p = first[i]; p <= last[i]; ++p)
      if (c->group[p] == p && !on_device(c, p)) return DITA_ERR_STATE;
  *n_out = n;
  return DITA_OK;
}

// Arguments of dita_state_change (and of its allocation-free variant).
int check_change_args(const dita_shape* shape, const void* o_new, const float* lse_new,
                      const void* o_prev, const float* lse_prev, int roll, const double* out) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_dev(o_new)) || (st = check_dev(o_prev)) || (st = check_dev(out))) return st;
  if (roll != 0 && roll != 1) return DITA_ERR_ARG;
  const size_t ob = state_o_bytes(*shape), lb = state_lse_bytes(*shape);
  if (overlaps(o_new, ob, o_prev, ob) || overlaps(out, 24, o_prev, ob) || overlaps(out, 24, o_new, ob))
    return DITA_ERR_ARG;
  if (roll) {
    if ((st = check_dev(lse_new)) || (st = check_dev(lse_prev))) return st;
    if (overlaps(lse_new, lb, lse_prev, lb) || overlaps(lse_prev, lb, o_new, ob) ||
        overlaps(o_prev, ob, lse_new, lb) || overlaps(out, 24, lse_prev, lb))
      return DITA_ERR_ARG;
  }
  return DITA_OK;
}

int ensure_events(dita_state_cache* c) {
  int st;
  if (!c->ev_fork && (st = hip_status(hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming))))
    return st;
  if (!c->ev_join && (st = hip_status(hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming))))
    return st;
  return DITA_OK;
}

}  // namespace

extern "C" {

const char* dita_status_str(int status) {
  switch (status) {
    case DITA_OK: return "ok";
    case DITA_ERR_ARG: return "invalid argument";
    case DITA_ERR_SHAPE: return "unsupported shape";
    case DITA_ERR_DTYPE: return "unsupported dtype";
    case DITA_ERR_STATE: return "reuse of a cache slot that holds no state";
    case DITA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case DITA_ERR_HIP: return "HIP runtime error";
    case DITA_ERR_SIZE: return "buffer too small";
    default: return "unknown status";
  }
}

int dita_last_hip_error(void) { return g_last_hip_error; }

int dita_version(void) { return 113; }

int dita_attn_partial(const dita_shape* shape, const void* q, const void* k, const void* v,
                      int64_t nk, void* o_p, float* lse_p, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  for (const void* p : {q, k, v, static_cast<const void*>(o_p), static_cast<const void*>(lse_p)})
    if ((st = check_dev(p))) return st;
  if (!nk_ok(*shape, nk)) return DITA_ERR_SHAPE;
  dita::AttnJobs jobs;
  jobs.job[0] = dita::AttnJob{k, v, o_p, lse_p, nk};
  return hip_status(launch_attn(*shape, q, jobs, 1, static_cast<hipStream_t>(stream)));
}

int dita_attn_launch_info(const dita_shape* shape, int n_blocks, int64_t nk,
                          dita_attn_layout* out) {
  int st = check_shape(shape);
  if (st) return st;
  if (!out) return DITA_ERR_ARG;
  if (shape->dtype != DITA_BF16) return DITA_ERR_DTYPE;
  if (n_blocks < 1 || n_blocks > DITA_MAX_PARTITIONS) return DITA_ERR_SHAPE;
  if (nk > 0 && !nk_ok(*shape, nk)) return DITA_ERR_SHAPE;
  const dita::AttnProblem pr = problem(*shape);
  dita::AttnLayout l{};
  if ((st = hip_status(dita::attn_bf16_layout(pr, n_blocks, nk, &l)))) return st;
  out->big_tiles = l.big;
  out->small_tiles = l.small;
  out->dual_tails = l.dual;
  out->workgroups = l.workgroups;
  out->split_units = l.units;
  out->split_tiles = l.rem;
  out->max_pieces = l.max_pieces;
  out->compute_units = l.cus;
  out->scratch_bytes = l.scratch;
  out->scratch_allocated = l.scratch_allocated;
  out->staged_pairs = l.stage_a;
  out->small_tiles_b = l.small_b;
  return DITA_OK;
}

int dita_state_merge(const dita_shape* shape, int P, const void* const* o_list,
                     const float* const* lse_list, void* o, float* lse, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (P < 1 || P > DITA_MAX_PARTITIONS) return DITA_ERR_SHAPE;
  if (!o_list || !lse_list) return DITA_ERR_ARG;
  if ((st = check_dev(o)) || (st = check_dev(lse))) return st;
  const size_t ob = state_o_bytes(*shape), lb = state_lse_bytes(*shape);
  dita::MergeSrc src{};
  for (int p = 0; p < P; ++p) {
    if ((st = check_dev(o_list[p])) || (st = check_dev(lse_list[p]))) return st;
    if (overlaps(o_list[p], ob, o, ob) || overlaps(lse_list[p], lb, lse, lb) ||
        overlaps(o_list[p], ob, lse, lb) || overlaps(lse_list[p], lb, o, ob))
      return DITA_ERR_ARG;
    src.o[p] = o_list[p];
    src.lse[p] = lse_list[p];
  }
  const int64_t rows = int64_t(shape->B) * shape->H * shape->Nq;
  return hip_status(dita::launch_merge(shape->dtype, shape->D, rows, P, src, o, lse,
                                       static_cast<hipStream_t>(stream)));
}

size_t dita_state_cache_bytes(const dita_shape* shape, int P) {
  if (check_shape(shape) || P < 1 || P > DITA_MAX_PARTITIONS) return 0;
  return size_t(P) * (align256(state_o_bytes(*shape)) + align256(state_lse_bytes(*shape)));
}

}  // extern "C"

namespace {

// Bytes of one compact slot and the offsets of its parts: int8 codes
// [rows, D], fp32 scales [rows], fp32 LSE [rows], each 256-byte aligned.
struct CompactLayout {
  size_t scale_off, lse_off, stride;
};
CompactLayout compact_layout(const dita_shape& s) {
  const size_t rows = size_t(s.B) * size_t(s.H) * size_t(s.Nq);
  CompactLayout l;
  l.scale_off = align256(rows * size_t(s.D));
  l.lse_off = l.scale_off + align256(rows * 4);
  l.stride = l.lse_off + align256(rows * 4);
  return l;
}

int cache_init(dita_state_cache** out, const dita_shape* shape, int P, int S, int C, bool pool,
               void* dev_buf, size_t bytes) {
  if (!out) return DITA_ERR_ARG;
  int st = check_shape(shape);
  if (st) return st;
  if (P < 1 || P > DITA_MAX_PARTITIONS || S < 1 || S > P) return DITA_ERR_SHAPE;
  if (C < 0 || C > P || S + C > DITA_MAX_PARTITIONS) return DITA_ERR_SHAPE;
  if (C > 0 && shape->dtype != DITA_BF16) return DITA_ERR_DTYPE;
  if ((st = check_dev(dev_buf))) return st;
  const size_t full = dita_state_cache_bytes(shape, S);
  const CompactLayout cl = compact_layout(*shape);
  const size_t need = full + size_t(C) * cl.stride;
  if (bytes < need) return DITA_ERR_SIZE;
  dita_state_cache* c = new (std::nothrow) dita_state_cache;
  if (!c) return DITA_ERR_ARG;
  c->shape = *shape;
  c->P = P;
  c->S = S;
  c->pool = pool;
  c->base = static_cast<char*>(dev_buf);
  c->bytes = bytes;
  c->o_bytes = state_o_bytes(*shape);
  c->lse_offset = align256(c->o_bytes);
  c->slot_stride = c->lse_offset + align256(state_lse_bytes(*shape));
  c->C = C;
  c->c_base = full;
  c->c_scale_off = cl.scale_off;
  c->c_lse_off = cl.lse_off;
  c->c_stride = cl.stride;
  for (int p = 0; p < DITA_MAX_PARTITIONS; ++p) {
    c->phys[p] = int16_t(pool || p >= P ? -1 : p);
    reset_slot(c, p);
  }
  c->ev_fork = nullptr;
  c->ev_join = nullptr;
  for (int k = 0; k < DITA_MAX_PARTITIONS; ++k) c->slot_ev[k] = -1;
  for (int e = 0; e <= DITA_MAX_PARTITIONS; ++e) {
    c->ev[e] = nullptr;
    c->ev_stream[e] = nullptr;
    c->ev_refs[e] = 0;
  }
  *out = c;
  return DITA_OK;
}

}  // namespace

extern "C" {

int dita_state_cache_init(dita_state_cache** out, const dita_shape* shape, int P, void* dev_buf,
                          size_t bytes) {
  return cache_init(out, shape, P, P, 0, false, dev_buf, bytes);
}

int dita_state_cache_init_pool(dita_state_cache** out, const dita_shape* shape, int P, int S,
                               void* dev_buf, size_t bytes) {
  return cache_init(out, shape, P, S, 0, true, dev_buf, bytes);
}

size_t dita_state_cache_bytes_compact(const dita_shape* shape, int S, int C) {
  if (check_shape(shape) || S < 1 || C < 0 || S + C > DITA_MAX_PARTITIONS) return 0;
  if (C > 0 && shape->dtype != DITA_BF16) return 0;
  return dita_state_cache_bytes(shape, S) + size_t(C) * compact_layout(*shape).stride;
}

int dita_state_cache_init_compact(dita_state_cache** out, const dita_shape* shape, int P, int S,
                                  int C, void* dev_buf, size_t bytes) {
  return cache_init(out, shape, P, S, C, true, dev_buf, bytes);
}

int dita_state_cache_compact(dita_state_cache* cache, int p, void* stream) {
  int st = check_slot(cache, p);
  if (st) return st;
  if (cache->C == 0) return DITA_ERR_STATE;
  if (!resident(cache, p) || cache->cphys[p] >= 0) return DITA_ERR_STATE;
  const int j = take_free_compact(cache);
  if (j < 0) return DITA_ERR_SIZE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int k = cache->phys[p];
  const uint64_t touched = slot_bit(k) | cslot_bit(cache, j);
  if ((st = slots_wait(cache, hs, touched))) return st;
  const dita_shape& s = cache->shape;
  const int64_t rows = int64_t(s.B) * s.H * s.Nq;
  if ((st = hip_status(dita::launch_compact_encode(s.D, phys_o(cache, k), phys_lse(cache, k),
                                                   cslot_codes(cache, j), cslot_scale(cache, j),
                                                   cslot_lse(cache, j), rows, hs))))
    return st;
  // The full slot goes back to the pool: its next owner waits for the encoding.
  if ((st = slots_mark(cache, hs, touched))) return st;
  release(cache, p);
  cache->cphys[p] = int16_t(j);
  return DITA_OK;
}

int dita_state_cache_compact_slot(const dita_state_cache* cache, int p, void** codes, float** scale,
                                  float** lse) {
  const int st = check_slot(cache, p);
  if (st) return st;
  const int j = cache->cphys[p];
  if (j < 0) return DITA_ERR_STATE;
  if (codes) *codes = cslot_codes(cache, j);
  if (scale) *scale = cslot_scale(cache, j);
  if (lse) *lse = cslot_lse(cache, j);
  return DITA_OK;
}

int dita_state_cache_format(const dita_state_cache* cache, int p, int* format) {
  const int st = check_slot(cache, p);
  if (st) return st;
  if (!format) return DITA_ERR_ARG;
  if (!cache->valid[p] || cache->group[p] != p)
    *format = DITA_STATE_NONE;
  else if (cache->on_host[p])
    *format = DITA_STATE_HOST;
  else if (cache->cphys[p] >= 0)
    *format = DITA_STATE_COMPACT;
  else
    *format = DITA_STATE_FULL;
  return DITA_OK;
}

int dita_state_cache_free(dita_state_cache* cache) {
  if (!cache) return DITA_OK;
  int st = DITA_OK;
  auto destroy = [&](hipEvent_t e) {
    if (!e) return;
    const int s2 = hip_status(hipEventDestroy(e));
    if (!st) st = s2;
  };
  destroy(cache->ev_fork);
  destroy(cache->ev_join);
  for (int e = 0; e <= DITA_MAX_PARTITIONS; ++e) destroy(cache->ev[e]);
  delete cache;
  return st;
}

int dita_state_cache_slot(const dita_state_cache* cache, int p, void** o, float** lse) {
  const int st = check_slot(cache, p);
  if (st) return st;
  if (cache->phys[p] < 0) return DITA_ERR_STATE;
  if (o) *o = slot_o(cache, p);
  if (lse) *lse = slot_lse(cache, p);
  return DITA_OK;
}

int dita_state_cache_store(dita_state_cache* cache, int p, const void* o, const float* lse,
                           int64_t step, void* stream) {
  int st = check_slot(cache, p);
  if (st) return st;
  if ((st = check_dev(o)) || (st = check_dev(lse))) return st;
  if (step < 0) return DITA_ERR_ARG;
  if (cache->group[p] != p || group_last(cache, p) != p) return DITA_ERR_STATE;
  const size_t lb = state_lse_bytes(cache->shape);
  if (overlaps(o, cache->o_bytes, cache->base, cache->bytes) ||
      overlaps(lse, lb, cache->base, cache->bytes))
    return DITA_ERR_ARG;
  uint64_t taken = 0;
  const int k = cache->phys[p] >= 0 ? cache->phys[p] : take_free(cache, &taken);
  if (k < 0) return DITA_ERR_SIZE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = slots_wait(cache, hs, slot_bit(k)))) return st;
  st = hip_status(dita::launch_copy_state(o, lse, phys_o(cache, k), phys_lse(cache, k),
                                          cache->o_bytes, lb, hs));
  if (st) return st;
  if ((st = slots_mark(cache, hs, slot_bit(k)))) return st;
  cache->phys[p] = int16_t(k);
  cache->cphys[p] = -1;
  forget_host(cache, p);
  cache->valid[p] = 1;
  cache->stamp[p] = step;
  return DITA_OK;
}

int dita_state_cache_load(const dita_state_cache* cache, int p, void* o, float* lse, void* stream) {
  int st = check_slot(cache, p);
  if (st) return st;
  if ((st = check_dev(o)) || (st = check_dev(lse))) return st;
  if (!cache->valid[p] || cache->group[p] != p || cache->cphys[p] >= 0) return DITA_ERR_STATE;
  const size_t lb = state_lse_bytes(cache->shape);
  if (overlaps(o, cache->o_bytes, cache->base, cache->bytes) ||
      overlaps(lse, lb, cache->base, cache->bytes))
    return DITA_ERR_ARG;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (cache->on_host[p]) {
    if ((st = hip_status(hipMemcpyAsync(o, cache->host_o[p], cache->o_bytes, hipMemcpyHostToDevice, hs))))
      return st;
    return hip_status(hipMemcpyAsync(lse, cache->host_lse[p], lb, hipMemcpyHostToDevice, hs));
  }
  // The ordering record of a pooled slot is bookkeeping, not the cache's state.
  dita_state_cache* mc = const_cast<dita_state_cache*>(cache);
  const uint64_t k = slot_bit(cache->phys[p]);
  if ((st = slots_wait(mc, hs, k))) return st;
  if ((st = hip_status(dita::launch_copy_state(slot_o(cache, p), slot_lse(cache, p), o, lse,
                                               cache->o_bytes, lb, hs))))
    return st;
  return slots_mark(mc, hs, k);
}

int dita_state_cache_invalidate(dita_state_cache* cache, int p) {
  if (!cache) return DITA_ERR_ARG;
  if (p == -1) {
    for (int i = 0; i < cache->P; ++i) reset_slot(cache, i);
    return DITA_OK;
  }
  const int st = check_slot(cache, p);
  if (st) return st;
  const int first = cache->group[p], last = group_last(cache, first);
  for (int i = first; i <= last; ++i) reset_slot(cache, i);
  return DITA_OK;
}

int dita_state_cache_info(const dita_state_cache* cache, int p, int* valid, int64_t* stamp) {
  const int st = check_slot(cache, p);
  if (st) return st;
  if (valid) *valid = cache->valid[p];
  if (stamp) *stamp = cache->stamp[cache->group[p]];
  return DITA_OK;
}

int dita_state_cache_shape(const dita_state_cache* cache, dita_shape* shape, int* P) {
  if (!cache) return DITA_ERR_ARG;
  if (shape) *shape = cache->shape;
  if (P) *P = cache->P;
  return DITA_OK;
}

int dita_state_cache_compose(dita_state_cache* cache, int first, int last, void* stream) {
  if (!cache) return DITA_ERR_ARG;
  if (first < 0 || last < first || last >= cache->P) return DITA_ERR_ARG;
  for (int p = first; p <= last; ++p) {
    if (!cache->valid[p]) return DITA_ERR_STATE;
    if (cache->group[p] < first || group_last(cache, cache->group[p]) > last) return DITA_ERR_ARG;
  }
  for (int p = first; p <= last; ++p)
    if (cache->group[p] == p && !on_device(cache, p)) return DITA_ERR_STATE;  // fetch it first
  int out_k = -1, src0 = -1;
  if (leaders_in(cache, first, last) > 1) {
    uint64_t taken = 0;
    if ((out_k = compose_output(cache, first, last, &taken, &src0)) < 0) return DITA_ERR_SIZE;
  }
  return compose_range(cache, first, last, out_k, src0, static_cast<hipStream_t>(stream), nullptr);
}

int dita_state_cache_compose_runs(dita_state_cache* cache, const uint8_t* reuse, void* stream,
                                  int* n_launched) {
  if (!cache || !reuse) return DITA_ERR_ARG;
  int first[DITA_MAX_PARTITIONS], last[DITA_MAX_PARTITIONS], n = 0;
  int st0 = plan_runs(cache, reuse, first, last, &n);
  if (st0) return st0;
  int out_k[DITA_MAX_PARTITIONS], src0[DITA_MAX_PARTITIONS];
  uint64_t taken = 0;
  for (int i = 0; i < n; ++i) {
    out_k[i] = src0[i] = -1;
    if (leaders_in(cache, first[i], last[i]) > 1 &&
        (out_k[i] = compose_output(cache, first[i], last[i], &taken, &src0[i])) < 0)
      return DITA_ERR_SIZE;
  }
  int launched = 0;
  for (int i = 0; i < n; ++i) {
    int l = 0;
    const int st = compose_range(cache, first[i], last[i], out_k[i], src0[i],
                                 static_cast<hipStream_t>(stream), &l);
    if (st) return st;
    launched += l;
  }
  if (n_launched) *n_launched = launched;
  return DITA_OK;
}

int dita_state_cache_group(const dita_state_cache* cache, int p, int* first, int* last) {
  const int st = check_slot(cache, p);
  if (st) return st;
  if (first) *first = cache->group[p];
  if (last) *last = group_last(cache, cache->group[p]);
  return DITA_OK;
}

int dita_state_cache_live(const dita_state_cache* cache, int* live) {
  if (!cache || !live) return DITA_ERR_ARG;
  int n = 0;
  for (int p = 0; p < cache->P; ++p) n += (cache->group[p] == p && cache->valid[p]) ? 1 : 0;
  *live = n;
  return DITA_OK;
}

int dita_state_cache_effective_mask(const dita_state_cache* cache, const uint8_t* reuse,
                                    uint8_t* out) {
  if (!cache || !reuse || !out) return DITA_ERR_ARG;
  uint8_t tmp[DITA_MAX_PARTITIONS];
  const int st = effective_mask(cache, reuse, tmp);
  if (st) return st;
  std::memcpy(out, tmp, size_t(cache->P));
  return DITA_OK;
}

int dita_plan_mask(const dita_plan* plan, const dita_state_cache* cache, int64_t step,
                   uint8_t* reuse_out) {
  if (!plan || !reuse_out || step < 0) return DITA_ERR_ARG;
  if (!dita::plan_valid(*plan)) return DITA_ERR_ARG;
  if (cache && cache->P != plan->P) return DITA_ERR_ARG;
  dita::plan_mask(*plan, step, cache ? cache->valid : nullptr, reuse_out);
  return DITA_OK;
}

int dita_mask_to_bits(const uint8_t* mask, int P, uint64_t* bits) {
  if (!mask || !bits || P < 1 || P > DITA_MAX_PARTITIONS) return DITA_ERR_ARG;
  uint64_t b = 0;
  for (int p = 0; p < P; ++p) {
    if (mask[p] > 1) return DITA_ERR_ARG;
    b |= uint64_t(mask[p]) << p;
  }
  *bits = b;
  return DITA_OK;
}

int dita_mask_from_bits(uint64_t bits, int P, uint8_t* mask) {
  if (!mask || P < 1 || P > DITA_MAX_PARTITIONS) return DITA_ERR_ARG;
  if (P < 64 && (bits >> P) != 0) return DITA_ERR_ARG;
  for (int p = 0; p < P; ++p) mask[p] = uint8_t((bits >> p) & 1);
  return DITA_OK;
}

int dita_plan_bits(const dita_plan* plan, const dita_state_cache* cache, int64_t step,
                   uint64_t* reuse_bits) {
  if (!reuse_bits) return DITA_ERR_ARG;
  uint8_t m[DITA_MAX_PARTITIONS];
  const int st = dita_plan_mask(plan, cache, step, m);
  if (st) return st;
  return dita_mask_to_bits(m, plan->P, reuse_bits);
}

int dita_attn_step(dita_state_cache* cache, const void* q, const void* const* k_list,
                   const void* const* v_list, const int64_t* nk_list, const uint8_t* reuse_mask,
                   int64_t step, void* o, float* lse, void* stream, dita_step_info* info) {
  return dita_attn_step_ex(cache, q, k_list, v_list, nk_list, reuse_mask, step, o, lse, stream,
                           nullptr, info);
}

int dita_attn_step_ex(dita_state_cache* cache, const void* q, const void* const* k_list,
                      const void* const* v_list, const int64_t* nk_list, const uint8_t* reuse_mask,
                      int64_t step, void* o, float* lse, void* stream, const dita_step_opts* opts,
                      dita_step_info* info) {
  if (!cache || !k_list || !v_list || !nk_list || !reuse_mask) return DITA_ERR_ARG;
  int st;
  if ((st = check_dev(q)) || (st = check_dev(o)) || (st = check_dev(lse))) return st;
  if (step < 0) return DITA_ERR_ARG;
  if (opts && (opts->reserved != 0 || opts->min_premerge < 0)) return DITA_ERR_ARG;
  const dita_shape& s = cache->shape;
  const int P = cache->P;
  const uint8_t* compose_next = opts ? opts->compose_next : nullptr;
  if (compose_next)
    for (int p = 0; p < P; ++p)
      if (compose_next[p] > 1) return DITA_ERR_ARG;
  const size_t ob = cache->o_bytes, lb = state_lse_bytes(s);
  if (overlaps(o, ob, cache->base, cache->bytes) || overlaps(lse, lb, cache->base, cache->bytes) ||
      overlaps(q, ob, cache->base, cache->bytes) || overlaps(o, ob, lse, lb))
    return DITA_ERR_ARG;

  uint8_t reuse[DITA_MAX_PARTITIONS];
  if ((st = effective_mask(cache, reuse_mask, reuse))) return st;
  // Physical slots: fresh partitions without one, and reused states that sit in
  // host memory (fetched back before the merge), take free slots.
  int16_t phys[DITA_MAX_PARTITIONS];
  uint64_t taken = 0;
  for (int p = 0; p < P; ++p) phys[p] = cache->phys[p];
  dita::AttnJobs jobs;
  int n_fresh = 0;
  double fresh_keys = 0.0;
  for (int p = 0; p < P; ++p) {
    if (reuse[p]) continue;
    if ((st = check_dev(k_list[p])) || (st = check_dev(v_list[p]))) return st;
    if (!nk_ok(s, nk_list[p])) return DITA_ERR_SHAPE;
    if (phys[p] < 0 && (phys[p] = int16_t(take_free(cache, &taken))) < 0) return DITA_ERR_SIZE;
    jobs.job[n_fresh++] =
        dita::AttnJob{k_list[p], v_list[p], phys_o(cache, phys[p]), phys_lse(cache, phys[p]), nk_list[p]};
    fresh_keys += double(nk_list[p]);
  }
  // Reused group states (leaders), in partition order; those on the host are fetched.
  int reused_heads[DITA_MAX_PARTITIONS], n_reused_heads = 0;
  int fetch[DITA_MAX_PARTITIONS], n_fetch = 0;
  for (int p = 0; p < P; ++p) {
    if (!reuse[p] || cache->group[p] != p) continue;
    reused_heads[n_reused_heads++] = p;
    if (cache->on_host[p]) {
      if (phys[p] < 0 && (phys[p] = int16_t(take_free(cache, &taken))) < 0) return DITA_ERR_SIZE;
      fetch[n_fetch++] = p;
    }
  }

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipStream_t side = opts ? static_cast<hipStream_t>(opts->side_stream) : nullptr;
  if (side == hs) side = nullptr;
  if (side) {
    // The side stream may write (o, lse) while the attention on `stream` still
    // reads Q and the fresh K/V: none of them may share memory with the output.
    const size_t esz = elem_size(s.dtype);
    const size_t row_bytes = size_t(s.B) * size_t(s.H) * size_t(s.D) * esz;
    if (overlaps(o, ob, q, ob) || overlaps(lse, lb, q, ob)) return DITA_ERR_ARG;
    for (int p = 0; p < P; ++p) {
      if (reuse[p]) continue;
      const size_t kb = row_bytes * size_t(nk_list[p]);
      if (overlaps(o, ob, k_list[p], kb) || overlaps(lse, lb, k_list[p], kb) ||
          overlaps(o, ob, v_list[p], kb) || overlaps(lse, lb, v_list[p], kb))
        return DITA_ERR_ARG;
    }
  }
  const int min_pre = opts && opts->min_premerge > 2 ? opts->min_premerge : 2;
  const bool premerge = side && n_fresh > 0 && n_reused_heads >= min_pre;
  const bool use_side = side && (premerge || n_fetch > 0);
  if (use_side && (st = ensure_events(cache))) return st;

  // Pooled slots this step writes (fresh, fetched) or reads (reused leaders).
  uint64_t touched = 0;
  for (int p = 0; p < P; ++p) {
    if (reuse[p] && cache->group[p] != p) continue;
    touched |= (!reuse[p] || cache->on_host[p]) ? slot_bit(phys[p]) : state_bit(cache, p);
  }
  if ((st = slots_wait(cache, hs, touched))) return st;

  if (info && info->ev_begin && (st = hip_status(hipEventRecord(static_cast<hipEvent_t>(info->ev_begin), hs))))
    return st;
  const int64_t rows = int64_t(s.B) * s.H * s.Nq;
  hipStream_t aux = use_side ? side : hs;
  if (use_side) {
    // The side stream starts after everything already on `stream` (earlier
    // writers of the reused slots and of the host copies, users of o/lse).
    if ((st = hip_status(hipEventRecord(cache->ev_fork, hs))) ||
        (st = hip_status(hipStreamWaitEvent(side, cache->ev_fork, 0))))
      return st;
  }
  for (int i = 0; i < n_fetch; ++i) {
    const int p = fetch[i];
    if ((st = hip_status(hipMemcpyAsync(phys_o(cache, phys[p]), cache->host_o[p], ob,
                                        hipMemcpyHostToDevice, aux))) ||
        (st = hip_status(hipMemcpyAsync(phys_lse(cache, phys[p]), cache->host_lse[p], lb,
                                        hipMemcpyHostToDevice, aux))))
      return st;
  }
  if (premerge) {
    // Merge the reused states into (o, lse) while the fresh attention runs.
    dita::MergeSrc pre{};
    int n_pre = 0;
    for (int i = 0; i < n_reused_heads; ++i) {
      const int p = reused_heads[i];
      if (cache->on_host[p]) {  // fetched into phys[p] above
        pre.o[n_pre] = phys_o(cache, phys[p]);
        pre.lse[n_pre] = phys_lse(cache, phys[p]);
        ++n_pre;
      } else {
        add_source(cache, pre, n_pre, p);
      }
    }
    if ((st = hip_status(dita::launch_merge(s.dtype, s.D, rows, n_reused_heads, pre, o, lse, side))))
      return st;
  }
  if (use_side && (st = hip_status(hipEventRecord(cache->ev_join, side)))) return st;
  if (n_fresh > 0 && (st = hip_status(launch_attn(s, q, jobs, n_fresh, hs)))) return st;
  if (info && info->ev_attn_end &&
      (st = hip_status(hipEventRecord(static_cast<hipEvent_t>(info->ev_attn_end), hs))))
    return st;
  // Recomputed groups dissolve; fresh slots take this step's stamp; fetched
  // states are resident again.
  for (int p = 0; p < P; ++p) {
    if (!reuse[p]) {
      cache->valid[p] = 1;
      cache->stamp[p] = step;
      cache->group[p] = int16_t(p);
      cache->phys[p] = phys[p];
      cache->cphys[p] = -1;
      forget_host(cache, p);
    }
  }
  for (int i = 0; i < n_fetch; ++i) {
    cache->phys[fetch[i]] = phys[fetch[i]];
    forget_host(cache, fetch[i]);
  }

  dita::MergeSrc src{};
  int n_src = 0;
  double src_bytes = 0.0;  // bytes of the states the final merge reads
  const double compact_bytes = double(rows) * double(s.D + 8);
  if (use_side && (st = hip_status(hipStreamWaitEvent(hs, cache->ev_join, 0)))) return st;
  if (premerge) {
    src.o[n_src] = o;  // the pre-merged reused states; the merge writes it in place
    src.lse[n_src] = lse;
    ++n_src;
    src_bytes += double(ob + lb);
  }
  // Composition ahead: after this step every partition holds a valid state on
  // the device, so the runs the next step reuses can be composed now.  The
  // largest run is composed by the final merge itself (its leaders are
  // consecutive sources there, and the group state comes from the same loads);
  // the others, and every run after a pre-merge, by merges of their own after
  // it.  A run whose group state would need a free slot that a pooled cache
  // lacks is left as it is.
  int run_first[DITA_MAX_PARTITIONS], run_last[DITA_MAX_PARTITIONS], n_runs = 0;
  int fused = -1, fused_out = -1, fused_src0 = -1;
  uint64_t taken_runs = taken;
  if (compose_next) {
    if ((st = plan_runs(cache, compose_next, run_first, run_last, &n_runs))) return st;
    int most = 1;
    for (int i = 0; i < n_runs && !premerge; ++i) {
      const int l = leaders_in(cache, run_first[i], run_last[i]);
      if (l > most) {
        most = l;
        fused = i;
      }
    }
    if (fused >= 0 &&
        (fused_out = compose_output(cache, run_first[fused], run_last[fused], &taken_runs,
                                    &fused_src0)) < 0)
      fused = -1;
  }
  dita::MergeGroup group{};
  for (int p = 0; p < P; ++p) {
    if (cache->group[p] != p || (premerge && reuse[p])) continue;
    src_bytes += cache->cphys[p] >= 0 ? compact_bytes : double(ob + lb);
    if (fused >= 0 && p == run_first[fused]) group.first = n_src;
    add_source(cache, src, n_src, p);
    if (fused >= 0 && p <= run_last[fused]) group.end = n_src;
  }
  if (fused >= 0) {
    group.o = phys_o(cache, fused_out);
    group.lse = phys_lse(cache, fused_out);
    // A group state written out of place goes to a slot from the pool.
    if ((st = slots_wait(cache, hs, slot_bit(fused_out)))) return st;
    touched |= slot_bit(fused_out);
  }
  if ((st = hip_status(dita::launch_merge(s.dtype, s.D, rows, n_src, src, o, lse, hs, group))))
    return st;
  if ((st = slots_mark(cache, hs, touched))) return st;
  int composed = 0;
  if (fused >= 0) {
    finish_compose(cache, run_first[fused], run_last[fused], fused_out);
    ++composed;
  }
  for (int i = 0; i < n_runs; ++i) {
    if (i == fused) continue;
    int out_k = -1, src0 = -1;
    if (leaders_in(cache, run_first[i], run_last[i]) > 1 &&
        (out_k = compose_output(cache, run_first[i], run_last[i], &taken_runs, &src0)) < 0)
      continue;
    if ((st = compose_range(cache, run_first[i], run_last[i], out_k, src0, hs, nullptr))) return st;
    ++composed;
  }
  if (info && info->ev_end && (st = hip_status(hipEventRecord(static_cast<hipEvent_t>(info->ev_end), hs))))
    return st;
  if (info) {
    info->n_fresh = n_fresh;
    info->n_reused = P - n_fresh;
    info->fresh_flops = 4.0 * double(s.B) * s.H * double(s.Nq) * fresh_keys * s.D;
    info->merge_sources = n_src;
    // The output, and the group state the final merge composed, if any.
    info->merge_bytes = src_bytes + double(ob + lb) * (fused >= 0 ? 2.0 : 1.0);
    info->premerge_sources = premerge ? n_reused_heads : 0;
    double pre_bytes = double(ob + lb);
    for (int i = 0; i < n_reused_heads; ++i)
      pre_bytes += cache->cphys[reused_heads[i]] >= 0 ? compact_bytes : double(ob + lb);
    info->premerge_bytes = premerge ? pre_bytes : 0.0;
    info->fetched = n_fetch;
    info->composed = composed;
  }
  return DITA_OK;
}

int dita_state_cache_offload(dita_state_cache* cache, int p, void* host_o, float* host_lse,
                             void* stream) {
  int st = check_slot(cache, p);
  if (st) return st;
  if (!host_o || !host_lse) return DITA_ERR_ARG;
  if (!resident(cache, p)) return DITA_ERR_STATE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t lb = state_lse_bytes(cache->shape);
  const uint64_t k = slot_bit(cache->phys[p]);
  if ((st = slots_wait(cache, hs, k))) return st;
  if ((st = hip_status(hipMemcpyAsync(host_o, slot_o(cache, p), cache->o_bytes,
                                      hipMemcpyDeviceToHost, hs))) ||
      (st = hip_status(hipMemcpyAsync(host_lse, slot_lse(cache, p), lb, hipMemcpyDeviceToHost, hs))))
    return st;
  // The slot goes back to the pool: its next owner waits for these copies.
  if ((st = slots_mark(cache, hs, k))) return st;
  cache->on_host[p] = 1;
  cache->host_o[p] = host_o;
  cache->host_lse[p] = host_lse;
  release(cache, p);
  return DITA_OK;
}

int dita_state_cache_fetch(dita_state_cache* cache, int p, void* stream) {
  int st = check_slot(cache, p);
  if (st) return st;
  if (!cache->valid[p] || cache->group[p] != p || !cache->on_host[p]) return DITA_ERR_STATE;
  uint64_t taken = 0;
  const int k = cache->phys[p] >= 0 ? cache->phys[p] : take_free(cache, &taken);
  if (k < 0) return DITA_ERR_SIZE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = slots_wait(cache, hs, slot_bit(k)))) return st;
  if ((st = hip_status(hipMemcpyAsync(phys_o(cache, k), cache->host_o[p], cache->o_bytes,
                                      hipMemcpyHostToDevice, hs))) ||
      (st = hip_status(hipMemcpyAsync(phys_lse(cache, k), cache->host_lse[p],
                                      state_lse_bytes(cache->shape), hipMemcpyHostToDevice, hs))))
    return st;
  if ((st = slots_mark(cache, hs, slot_bit(k)))) return st;
  cache->phys[p] = int16_t(k);
  forget_host(cache, p);
  return DITA_OK;
}

int dita_state_cache_residency(const dita_state_cache* cache, int* on_device, int* on_host,
                               int* free_slots) {
  if (!cache) return DITA_ERR_ARG;
  int dev = 0, host = 0, full = 0;
  for (int p = 0; p < cache->P; ++p) {
    if (!cache->valid[p] || cache->group[p] != p) continue;
    if (cache->on_host[p])
      ++host;
    else
      ++dev;
    if (cache->phys[p] >= 0 && !cache->on_host[p] && cache->cphys[p] < 0) ++full;
  }
  if (on_device) *on_device = dev;
  if (on_host) *on_host = host;
  if (free_slots) *free_slots = cache->S - full;
  return DITA_OK;
}

int dita_state_contrib(const dita_shape* shape, int P, const float* const* lse_list,
                       const float* lse, double* w_out, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (P < 1 || P > DITA_MAX_PARTITIONS) return DITA_ERR_SHAPE;
  if (!lse_list) return DITA_ERR_ARG;
  if ((st = check_dev(lse)) || (st = check_dev(w_out))) return st;
  dita::LseList src;
  for (int p = 0; p < P; ++p) {
    if ((st = check_dev(lse_list[p]))) return st;
    src.lse[p] = lse_list[p];
  }
  const int64_t rows = int64_t(shape->B) * shape->H * shape->Nq;
  return hip_status(dita::launch_contrib(P, src, lse, rows, w_out, static_cast<hipStream_t>(stream)));
}

int dita_state_cache_contrib(const dita_state_cache* cache, const float* lse, double* w_out,
                             void* stream) {
  if (!cache) return DITA_ERR_ARG;
  int st;
  if ((st = check_dev(lse)) || (st = check_dev(w_out))) return st;
  const float* lses[DITA_MAX_PARTITIONS];
  uint64_t touched = 0;
  for (int p = 0; p < cache->P; ++p) {
    if (!on_device(cache, p) || group_last(cache, p) != p) return DITA_ERR_STATE;
    lses[p] = state_lse(cache, p);
    touched |= state_bit(cache, p);
  }
  if ((st = check_shape(&cache->shape))) return st;
  dita_state_cache* mc = const_cast<dita_state_cache*>(cache);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = slots_wait(mc, hs, touched))) return st;
  if ((st = dita_state_contrib(&cache->shape, cache->P, lses, lse, w_out, stream))) return st;
  return slots_mark(mc, hs, touched);
}

int dita_state_change(const dita_shape* shape, const void* o_new, const float* lse_new,
                      void* o_prev, float* lse_prev, int roll, double* out, void* stream) {
  const int st = check_change_args(shape, o_new, lse_new, o_prev, lse_prev, roll, out);
  if (st) return st;
  // Partial sums of the workgroups: stream-ordered scratch from HIP's pool,
  // returned to it once the finishing kernel has read it.
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t ob = state_o_bytes(*shape), lb = state_lse_bytes(*shape);
  const size_t scratch_bytes = size_t(2) * size_t(dita::change_groups(ob)) * sizeof(double);
  void* part = nullptr;
  int s2 = hip_status(hipMallocAsync(&part, scratch_bytes, hs));
  if (s2) return s2;
  s2 = hip_status(dita::launch_change(shape->dtype, o_new, o_prev, ob, lse_new, lse_prev,
                                      roll ? lb : 0, roll, static_cast<double*>(part), out, hs));
  const int s3 = hip_status(hipFreeAsync(part, hs));
  return s2 ? s2 : s3;
}

}  // extern "C"

namespace {

// Scratch of dita_state_change_noalloc: the partial sums of the change
// statistic's workgroups (two doubles each; the grid never exceeds
// dita::kChangeMaxGroups workgroups, so 16 KB covers every state size).  Each
// GPU holds its own copy until the process ends; host code reaches it only
// through the per-device address from hipGetSymbolAddress.
constexpr int kNoAllocScratchDoubles = 2 * dita::kChangeMaxGroups;
static __device__ __align__(256) double scratch[kNoAllocScratchDoubles];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
int scratch_on_current_device(double** out) {
  int dev = 0;
  int st = hip_status(hipGetDevice(&dev));
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return DITA_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))))) return st;
    if (!ptr) return DITA_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<double*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return DITA_OK;
}

}  // namespace

extern "C" {

int dita_state_change_noalloc(const dita_shape* shape, const void* o_new, const float* lse_new,
                              void* o_prev, float* lse_prev, int roll, double* out, void* stream) {
  int st = check_change_args(shape, o_new, lse_new, o_prev, lse_prev, roll, out);
  if (st) return st;
  const size_t ob = state_o_bytes(*shape), lb = state_lse_bytes(*shape);
  if (2 * dita::change_groups(ob) > kNoAllocScratchDoubles) return DITA_ERR_SIZE;
  double* part = nullptr;
  if ((st = scratch_on_current_device(&part))) return st;
  return hip_status(dita::launch_change(shape->dtype, o_new, o_prev, ob, lse_new, lse_prev,
                                        roll ? lb : 0, roll, part, out,
                                        static_cast<hipStream_t>(stream)));
}

int dita_planner_mask_cache(const dita_planner* planner, const dita_state_cache* cache,
                            int64_t step, uint8_t* reuse_out, double* err_out) {
  if (!cache) return DITA_ERR_ARG;
  int64_t stamp[DITA_MAX_PARTITIONS];
  for (int p = 0; p < cache->P; ++p) stamp[p] = cache->stamp[cache->group[p]];
  return dita_planner_mask(planner, step, cache->valid, stamp, reuse_out, err_out);
}

int dita_event_create(void** event) {
  if (!event) return DITA_ERR_ARG;
  hipEvent_t e = nullptr;
  const int st = hip_status(hipEventCreate(&e));
  if (st) return st;
  *event = e;
  return DITA_OK;
}

int dita_event_destroy(void* event) {
  if (!event) return DITA_OK;
  return hip_status(hipEventDestroy(static_cast<hipEvent_t>(event)));
}

int dita_event_record(void* event, void* stream) {
  if (!event) return DITA_ERR_ARG;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream)));
}

int dita_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return DITA_ERR_ARG;
  int st = hip_status(hipEventSynchronize(static_cast<hipEvent_t>(stop)));
  if (st) return st;
  return hip_status(
      hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)));
}

}  // extern "C"
