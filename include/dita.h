/*
 * dita.h -- C ABI of the selective attention-state reuse library for MI355X (gfx950).
 *
 * One rank owns a query partition Q and attends to P key/value context
 * partitions (K_p, V_p).  For every partition the rank either computes a
 * fresh attention state (O_p, LSE_p) or reuses the state cached at an
 * earlier denoising step; all P states are then merged exactly by their
 * log-sum-exp weights.  Method: the web page "DiTango: Cost-Effective
 * Parallel Diffusion Generation with Selective Attention State Reuse"
 * (gist.science, paper 2607.15650), section Methodology:
 *   - "2. State-Centric Parallel Runtime" > "State Composition": a state is an
 *     output plus its log-sum-exp; states compose associatively and
 *     commutatively; composed states are cached instead of raw K/V.
 *   - "1. Anchor-Guided Selection Planner": each partition is computed fresh
 *     or its historical state is reused; anchor steps recompute everything;
 *     the local partition is always computed.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every function returns an int status (dita_status).  Nothing throws.
 *  - Every argument is validated before any HIP call or kernel launch; on an
 *    error nothing is launched and no output, slot or metadata changes.  A
 *    HIP runtime failure (DITA_ERR_HIP) part-way through a call that enqueues
 *    several operations may leave the earlier ones enqueued (a step that fails
 *    after its attention launch has already recorded the fresh states in the
 *    cache metadata); the stream should then be treated as failed.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and is asynchronous: no call synchronises the host.  Faults of
 *    the kernels surface at the caller's next synchronisation.
 *  - The caller owns every device buffer, the state-cache buffer included.
 *    The library owns only the host-side cache handle (and its HIP events),
 *    and the transient scratch of dita_state_change, taken from HIP's
 *    stream-ordered allocator and returned within the call.
 *  - Layouts are contiguous row-major: Q and O are [B, H, Nq, D]; K_p and
 *    V_p are [B, H, Nk_p, D]; LSE arrays are float32 [B, H, Nq].  O and O_p
 *    have the input dtype; LSE is always float32 and uses the natural log.
 *  - Device pointers must be 16-byte aligned.  D is 64 or 128.  B*H <= 65535,
 *    1 <= Nq, Nk <= 2^30, Nk * D * sizeof(dtype) < 2^31 (one head's K or V
 *    slice), 1 <= P <= DITA_MAX_PARTITIONS.
 *  - O_p is normalised by its own partition's softmax denominator (each row
 *    is a convex combination of V_p's rows); the unnormalised output is
 *    exp(LSE_p) * O_p.
 *  - Attention is bidirectional (no mask) with softmax scale `scale`
 *    (<= 0 selects 1/sqrt(D)).
 *  - Non-finite inputs are not supported and not checked.
 *  - A cache handle is not thread-safe; calls that share one must be
 *    serialised by the caller.
 */
#ifndef DITA_H
#define DITA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DITA_MAX_PARTITIONS 64

typedef enum {
  DITA_OK = 0,
  DITA_ERR_ARG = 1,    /* null pointer, or an integer argument out of range      */
  DITA_ERR_SHAPE = 2,  /* unsupported shape (D, B*H, Nq, Nk, P)                  */
  DITA_ERR_DTYPE = 3,  /* unknown dtype                                          */
  DITA_ERR_STATE = 4,  /* reuse of a slot that holds no state                    */
  DITA_ERR_ALIGN = 5,  /* a device pointer is not 16-byte aligned                */
  DITA_ERR_HIP = 6,    /* a HIP runtime call failed; see dita_last_hip_error()   */
  DITA_ERR_SIZE = 7    /* a caller buffer is smaller than required               */
} dita_status;

typedef enum { DITA_F32 = 0, DITA_BF16 = 1 } dita_dtype;

/* Shape of one rank's attention problem. */
typedef struct {
  int32_t B;      /* batch                                   */
  int32_t H;      /* heads                                   */
  int32_t D;      /* head dimension: 64 or 128               */
  int32_t dtype;  /* dita_dtype of Q, K, V, O                */
  int64_t Nq;     /* query rows of the rank's partition      */
  float scale;    /* softmax scale; <= 0 selects 1/sqrt(D)   */
} dita_shape;

/* Human-readable name of a status code (static storage; never NULL). */
const char* dita_status_str(int status);

/* The hipError_t of the most recent DITA_ERR_HIP on the calling thread (0 if none). */
int dita_last_hip_error(void);

/* Library ABI version (major * 100 + minor). */
int dita_version(void);

/*
 * dita_attn_partial -- fresh attention state of Q against one K/V partition.
 * Page section: State-Centric Parallel Runtime > State Composition (a state
 * is an output plus its log-sum-exp).
 *
 *   S = scale * Q K^T;  LSE_p = ln sum_j exp(S_ij);  O_p = exp(S - LSE_p) V
 *
 * q      [in]  device, [B, H, Nq, D] dtype
 * k, v   [in]  device, [B, H, nk, D] dtype
 * nk     [in]  keys in the partition, >= 1
 * o_p    [out] device, [B, H, Nq, D] dtype (may not alias q, k, v)
 * lse_p  [out] device, [B, H, Nq] float32
 * bf16 runs on MFMA with fp32 accumulation; f32 keeps every step in fp32.
 */
int dita_attn_partial(const dita_shape* shape, const void* q, const void* k, const void* v,
                      int64_t nk, void* o_p, float* lse_p, void* stream);

/*
 * Work layout of the bf16 attention kernel (dita_attn_partial, and the fresh
 * blocks of one dita_attn_step, which share one launch).  Each workgroup takes
 * a 512-query tile of one (batch, head, block) against all of the block's
 * keys; rows past the last whole 512-row tile go into one more such tile, into
 * 256-row tiles, or (at most 128 of them, blocks of one key length) into
 * 256-row workgroups that each take the tail rows of two (batch, head, block)
 * pairs, one per half, whichever finishes sooner.  In the staged layout all
 * 512-row tiles run before all 256-row tiles, and some pairs trade one 512-row
 * tile for two 256-row tiles so that the 512-row tiles fill whole rounds of
 * the device's compute units (staged_pairs below).  When the 512-row tiles do
 * not fill the last round of the device's compute units, the tiles of that
 * round are instead computed in pieces along the key axis: split_units
 * workgroups each take an equal share of those tiles' key-tile iterations
 * (at most two segments, computed one after the other), and the last piece of a
 * tile to finish combines the pieces by their LSEs.  That is the pages' state
 * composition applied to key sub-ranges of one partition (State-Centric
 * Parallel Runtime > State Composition): exact up to rounding, and the
 * result does not depend on which piece finishes last.
 *
 * The pieces live in a device scratch that the library allocates on the first
 * such launch on a device (scratch_allocated bytes: 2 x 256 x 264 KiB + 16
 * KiB, about 138 MB, the most any launch uses) and keeps, at the same address,
 * until the process ends.  Launches that use it from different streams are
 * ordered by an event.  A launch under stream capture uses it without
 * waiting or recording (the caller orders the graph's replays against other
 * attention calls on that device, e.g. by replaying on the stream they use);
 * one captured before the scratch exists runs without the split.  Blocks of
 * unequal key lengths are not split.
 */
typedef struct {
  int32_t big_tiles;        /* 512-row tiles per (batch, head, block)                     */
  int32_t small_tiles;      /* 256-row tiles per (batch, head, block), after the 512-row  */
  int32_t dual_tails;       /* 1: each 256-row workgroup takes the tails of two pairs     */
  int64_t workgroups;       /* grid size                                                  */
  int32_t split_units;      /* key-split units; 0: no split                               */
  int32_t split_tiles;      /* 512-row tiles computed in pieces                           */
  int32_t max_pieces;       /* most pieces of one split tile                              */
  int32_t compute_units;    /* of the current device                                      */
  int64_t scratch_bytes;    /* key-split scratch the launch uses                          */
  int64_t scratch_allocated;/* device scratch the library holds for splits (per device)   */
  int32_t staged_pairs;     /* >= 0: staged layout, all 512-row tiles dispatched before   */
                            /* all 256-row tiles; the first staged_pairs pairs have       */
                            /* big_tiles and small_tiles, the others big_tiles - 1 and    */
                            /* small_tiles_b.  -1: per-pair order (or no 256-row tiles)   */
  int32_t small_tiles_b;    /* staged layout: 256-row tiles of the other pairs            */
} dita_attn_layout;

/*
 * dita_attn_launch_info -- the layout above for n_blocks (1..DITA_MAX_PARTITIONS)
 * fresh blocks of nk keys each (nk <= 0: blocks of unequal lengths) of a bf16
 * problem, on the current device.  Host computation and a device-attribute
 * query; launches nothing.  DITA_ERR_DTYPE for fp32 problems (their kernel has
 * no tiles of this kind).
 */
int dita_attn_launch_info(const dita_shape* shape, int n_blocks, int64_t nk,
                          dita_attn_layout* out);

/*
 * dita_state_merge -- exact LSE-weighted composition of P attention states.
 * Page section: State-Centric Parallel Runtime > State Composition
 * (associative, commutative composition of states).
 *
 *   M = max_p LSE_p;  w_p = exp(LSE_p - M);  L = sum_p w_p
 *   O = sum_p (w_p / L) O_p;  LSE = M + ln L
 * A state whose LSE is -inf has weight 0; rows where every LSE_p is -inf
 * produce O = 0 and LSE = -inf.
 *
 * P         [in]  1..DITA_MAX_PARTITIONS
 * o_list    [in]  host array of P device pointers, each [B, H, Nq, D] dtype
 * lse_list  [in]  host array of P device pointers, each [B, H, Nq] float32
 * o, lse    [out] device, [B, H, Nq, D] dtype and [B, H, Nq] float32; they
 *                 may alias none of the inputs
 */
int dita_state_merge(const dita_shape* shape, int P, const void* const* o_list,
                     const float* const* lse_list, void* o, float* lse, void* stream);

/*
 * State cache -- device-resident per-partition (O_p, LSE_p) slots.
 * Page section: State-Centric Parallel Runtime > State Composition (cache
 * composed states instead of raw K/V) and > Pipeline Orchestration ("reuse"
 * operations load cached states).
 *
 * The caller allocates `bytes >= dita_state_cache_bytes(shape, P)` of device
 * memory (16-byte aligned; 256 recommended) and keeps it alive while the
 * handle exists.  Slot p holds O_p ([B, H, Nq, D] dtype) followed by LSE_p
 * ([B, H, Nq] float32), each at a 256-byte aligned offset.  Host metadata per
 * slot: valid (0/1), stamp (the step that last wrote it, -1 if never) and the
 * group the partition belongs to.
 *
 * Groups (page section: State-Centric Parallel Runtime > Dynamic Group
 * Compose -- cached states are merged recursively into coarser groups).  A
 * group is a contiguous range [first, last] of partitions whose states have
 * been composed into one state held in slot `first` (the leader); the other
 * member slots hold nothing of their own.  Every partition starts as a group
 * of one.  A group's stamp is the oldest stamp among the states composed into
 * it and is reported for every member.  Rules: a group is reused by a step
 * only when every member is marked reuse, otherwise every member is computed
 * fresh and the group dissolves into groups of one; store into any partition
 * of a group of two or more, and load from a member other than the leader,
 * return DITA_ERR_STATE; invalidating any member invalidates and dissolves
 * the whole group.
 */
typedef struct dita_state_cache dita_state_cache;

/* Device bytes a cache of P slots needs; 0 if the shape or P is invalid. */
size_t dita_state_cache_bytes(const dita_shape* shape, int P);

/* Create a handle over `dev_buf`; all slots start invalid.  *out is set only on DITA_OK.
 * Partition p owns physical slot p for the handle's lifetime. */
int dita_state_cache_init(dita_state_cache** out, const dita_shape* shape, int P, void* dev_buf,
                          size_t bytes);

/*
 * A pooled cache: P partitions share S <= P physical slots (bytes >=
 * dita_state_cache_bytes(shape, S)).  A partition holds a slot only while its
 * own state is on the device; composing a group, moving a state to the host,
 * or invalidating it returns the slot to the pool, and storing, computing or
 * fetching a state takes the lowest free one (DITA_ERR_SIZE, before any
 * launch, when none is free).  Page section: State-Centric Parallel Runtime >
 * Dynamic Group Compose (composition relieves memory pressure) -- with a pool,
 * the states a cache no longer holds are device memory the next state can use.
 *
 * Stream order of a pooled cache: because the library moves physical slots
 * between partitions, it orders the device work on each slot itself.  Every
 * call that enqueues work on pooled slots (store, load, offload, fetch,
 * compose, compose_runs, the steps, dita_state_cache_contrib) makes its
 * stream wait for the last work enqueued on each slot it touches when that
 * work was enqueued on another stream (hipStreamWaitEvent on an event the
 * handle records; events are created on first use and destroyed by
 * dita_state_cache_free).  So calls on one pooled handle may use different
 * streams: the work on any one slot runs in call order.  Work the caller
 * enqueues itself on slot memory (through dita_state_cache_slot) is outside
 * this order.  In a cache made by dita_state_cache_init, partition p owns
 * slot p; ordering calls on different streams is then the caller's concern,
 * as for any device buffer.
 */
int dita_state_cache_init_pool(dita_state_cache** out, const dita_shape* shape, int P, int S,
                               void* dev_buf, size_t bytes);

/*
 * Move group leader p's state to caller host memory (pinned memory --
 * hipHostMalloc -- lets the copies overlap other work): host_o holds
 * B*H*Nq*D elements of the dtype, host_lse B*H*Nq floats; both must stay
 * allocated, and must not be written, until the state is fetched, stored over
 * or invalidated.  Stream-ordered device-to-host copies; in a pooled cache the
 * slot returns to the pool.  The state stays valid: a step that reuses it, or
 * dita_state_cache_fetch, copies it back; when that happens on another stream
 * the caller orders it after this call's stream.  Page section: State-Centric
 * Parallel Runtime > Pipeline Orchestration ("reuse" operations load cached
 * states).  DITA_ERR_STATE unless p leads a valid group held on the device.
 */
int dita_state_cache_offload(dita_state_cache* cache, int p, void* host_o, float* host_lse,
                             void* stream);

/*
 * Compact states.  Page section: Significance and Claims (the memory held by
 * cached states is the method's stated limitation; cache compression is its
 * future work).  The page gives no format; this one keeps a bf16 state's
 * output as int8 codes with one float32 scale per row (row = one query of one
 * head), the LSE exactly:
 *   a = max_d |O[r, d]|;  scale[r] = a / 127;
 *   code[r, d] = round-half-even(O[r, d] * 127 / a) in [-127, 127]
 * (a row of zeros: scale 0, codes 0), each a float32 operation rounded once,
 * so the encoding is reproducible bit for bit.  A merge uses code * scale
 * (one float32 product), within scale/2 = a/254 of the stored bf16 value.
 * Bytes per row: D + 8 against 2D + 4 (136 against 260 at D = 128).
 *
 * A compact cache is a pooled cache (see dita_state_cache_init_pool) with S
 * full and C compact physical slots in one buffer of
 * dita_state_cache_bytes_compact(shape, S, C) bytes; bf16 only
 * (DITA_ERR_DTYPE otherwise), 1 <= S <= P, 0 <= C <= P, S + C <= 64.  Layout:
 * the S full slots as in dita_state_cache_bytes(shape, S), then C compact
 * slots, each int8 codes [B, H, Nq, D], float32 scales [B, H, Nq] and float32
 * LSE [B, H, Nq], every part at a 256-byte aligned offset.
 *
 * dita_state_cache_compact: encode group leader p's state (held in a full
 *   device slot) into a free compact slot and return the full slot to the
 *   pool (DITA_ERR_SIZE if no compact slot is free; DITA_ERR_STATE if p holds
 *   no full device state or the cache has no compact slots).  Stream-ordered;
 *   reads 2D + 4 bytes and writes D + 8 bytes per row.
 * A compact state is used as it is: steps that reuse it and compositions
 * that include it read its codes and scales in the merge (a composition's
 * result is a full state, written in place into a member's full slot, or into
 * a free one -- DITA_ERR_SIZE, before any launch, if none); a step that
 * recomputes it, or a store, replaces it with a full state and frees the
 * compact slot.  dita_state_cache_load, _offload and _slot return
 * DITA_ERR_STATE for a compact state; dita_state_cache_compact_slot gives its
 * device parts.  Residency counts compact states as on the device; the free
 * slots it reports are full ones.
 */
size_t dita_state_cache_bytes_compact(const dita_shape* shape, int S, int C);
int dita_state_cache_init_compact(dita_state_cache** out, const dita_shape* shape, int P, int S,
                                  int C, void* dev_buf, size_t bytes);
int dita_state_cache_compact(dita_state_cache* cache, int p, void* stream);
/* Device parts of p's compact state (any output pointer may be NULL); DITA_ERR_STATE unless
 * p's state is compact.  codes: int8 [B, H, Nq, D]; scale, lse: float32 [B, H, Nq]. */
int dita_state_cache_compact_slot(const dita_state_cache* cache, int p, void** codes, float** scale,
                                  float** lse);
/* Where partition p's own state is: DITA_STATE_NONE (invalid, or a member other than its
 * group's leader), _FULL (a full device slot), _COMPACT, or _HOST. */
enum { DITA_STATE_NONE = 0, DITA_STATE_FULL = 1, DITA_STATE_COMPACT = 2, DITA_STATE_HOST = 3 };
int dita_state_cache_format(const dita_state_cache* cache, int p, int* format);

/* Copy an offloaded state back into a device slot (DITA_ERR_SIZE if none is free). */
int dita_state_cache_fetch(dita_state_cache* cache, int p, void* stream);

/* Valid states (group leaders) on the device and on the host, and physical slots not holding one. */
int dita_state_cache_residency(const dita_state_cache* cache, int* on_device, int* on_host,
                               int* free_slots);

/* Destroy a handle (NULL is accepted).  Never frees dev_buf. */
int dita_state_cache_free(dita_state_cache* cache);

/* Device addresses of partition p's slot (either output pointer may be NULL).
 * DITA_ERR_STATE in a pooled cache when p holds no slot. */
int dita_state_cache_slot(const dita_state_cache* cache, int p, void** o, float** lse);

/* Copy a state into slot p (stream-ordered copy kernel) and mark it valid with `step`.
 * DITA_ERR_STATE if p belongs to a group of two or more partitions. */
int dita_state_cache_store(dita_state_cache* cache, int p, const void* o, const float* lse,
                           int64_t step, void* stream);

/* Copy slot p out to caller buffers (for a group leader: the group's state).
 * DITA_ERR_STATE if the slot is invalid or p is a group member other than the leader. */
int dita_state_cache_load(const dita_state_cache* cache, int p, void* o, float* lse, void* stream);

/* Mark slot p invalid, with every other member of its group (p = -1: every
 * slot); the group dissolves.  Device memory is untouched. */
int dita_state_cache_invalidate(dita_state_cache* cache, int p);

/* Read slot p's metadata (either output pointer may be NULL). */
int dita_state_cache_info(const dita_state_cache* cache, int p, int* valid, int64_t* stamp);

/* Cache geometry: P, and the shape it was created with. */
int dita_state_cache_shape(const dita_state_cache* cache, dita_shape* shape, int* P);

/*
 * Compose the cached states of partitions first..last into one group state,
 * written in place into slot `first` by the LSE merge kernel (groups already
 * inside the range enter as the single states they are, so composition is
 * recursive).  Page section: State-Centric Parallel Runtime > Dynamic Group
 * Compose.  Reads the range's leader slots and writes one state: with n
 * leaders, (n + 1) * (B*H*Nq*(D*size + 4)) bytes; no launch when the range
 * already is one group.
 * Errors: DITA_ERR_ARG unless 0 <= first <= last < P, or when a group
 * straddles the range; DITA_ERR_STATE when a partition in it holds no state.
 */
int dita_state_cache_compose(dita_state_cache* cache, int first, int last, void* stream);

/*
 * Compose ahead of a step: for every maximal run of partitions that `reuse`
 * (P bytes, 0/1 -- typically the next step's mask) marks for reuse, compose
 * the run into one group, leaving out groups that reach outside the run (a
 * step recomputes those whole).  Runs that already are one group, or hold one
 * partition, are left as they are.  A step with that mask then reads one state
 * per run.  *n_launched (nullable) receives the number of merge launches.
 * DITA_ERR_STATE if `reuse` marks an invalid slot; DITA_ERR_ARG for values
 * other than 0/1.
 */
int dita_state_cache_compose_runs(dita_state_cache* cache, const uint8_t* reuse, void* stream,
                                  int* n_launched);

/* The group [*first, *last] that holds partition p (either output may be NULL). */
int dita_state_cache_group(const dita_state_cache* cache, int p, int* first, int* last);

/* Number of states the cache holds: valid group leaders (a lone partition leads its own group). */
int dita_state_cache_live(const dita_state_cache* cache, int* live);

/*
 * The reuse mask a step applies for the caller's mask `reuse` (P bytes, 0/1):
 * equal to `reuse` except that a group with any member marked fresh is
 * computed fresh whole.  The caller must supply K/V for every partition whose
 * entry in `out` is 0.  DITA_ERR_STATE if `reuse` marks an invalid slot.
 */
int dita_state_cache_effective_mask(const dita_state_cache* cache, const uint8_t* reuse,
                                    uint8_t* out);

/*
 * Reuse-mask planner (host only, integer arithmetic, deterministic).
 * Page section: 1. Anchor-Guided Selection Planner -- anchor steps recompute
 * every partition; the local partition is always computed; the rest are
 * computed or reused per the policy.  The page prints no selection formula;
 * the policies are fixed schedules:
 *   DITA_PLAN_DIST      fresh iff |p - q| <= radius
 *   DITA_PLAN_KNEAREST  fresh iff p is among the k_nearest partitions closest
 *                       to q, ordered by (|p - q|, p)
 *   DITA_PLAN_RANDOM    one SplitMix64 stream per step, seeded with
 *                       (seed << 32) ^ step; P draws for p = 0..P-1 in order;
 *                       reuse iff the draw's top bit is 1
 *   DITA_PLAN_RAMP      fresh iff |p - q| <= r(step), r linear from `radius`
 *                       at step 0 to `radius_end` at total_steps-1, rounded
 *                       half up, clamped outside the schedule
 * Overrides (fresh): p == q; anchor_period > 0 and step % anchor_period == 0;
 * a slot that is not valid in `cache` (when cache is non-NULL).
 */
enum { DITA_PLAN_DIST = 0, DITA_PLAN_KNEAREST = 1, DITA_PLAN_RANDOM = 2, DITA_PLAN_RAMP = 3 };

typedef struct {
  int32_t P;              /* partitions, 1..DITA_MAX_PARTITIONS        */
  int32_t q;              /* the rank's local partition, 0..P-1        */
  int32_t policy;         /* DITA_PLAN_*                               */
  int32_t radius;         /* DIST radius; RAMP radius at step 0, >= 0  */
  int32_t radius_end;     /* RAMP radius at the last step, >= 0        */
  int32_t k_nearest;      /* KNEAREST count, >= 0                      */
  int32_t anchor_period;  /* > 0: every anchor_period-th step is fresh */
  int32_t total_steps;    /* RAMP schedule length, >= 1                */
  uint64_t seed;          /* RANDOM seed                               */
} dita_plan;

/* reuse_out [out, host]: P bytes, 1 = reuse the cached state, 0 = compute fresh. */
int dita_plan_mask(const dita_plan* plan, const dita_state_cache* cache, int64_t step,
                   uint8_t* reuse_out);

/*
 * The same mask as a 64-bit word: bit p set = partition p reused (bits >= P
 * clear).  dita_mask_to_bits / dita_mask_from_bits convert between the two
 * encodings (P in 1..DITA_MAX_PARTITIONS; mask bytes must be 0 or 1).
 */
int dita_plan_bits(const dita_plan* plan, const dita_state_cache* cache, int64_t step,
                   uint64_t* reuse_bits);
int dita_mask_to_bits(const uint8_t* mask, int P, uint64_t* bits);
int dita_mask_from_bits(uint64_t bits, int P, uint8_t* mask);

/*
 * dita_attn_step -- one rank-step of selective state reuse.
 * Page sections: 1. Anchor-Guided Selection Planner (per-partition compute or
 * reuse) and 2. State-Centric Parallel Runtime > State Composition.
 *
 * For every p with reuse_mask[p] == 0 the fresh state of Q against
 * (k_list[p], v_list[p]) is written straight into cache slot p (one grouped
 * launch for all fresh partitions) and the slot is stamped with `step`; slots
 * with reuse_mask[p] == 1 are left as they are and must be valid.  Composed
 * groups are reused or recomputed whole (see the cache's group rules and
 * dita_state_cache_effective_mask).  Then the states of all groups are merged
 * into (o, lse).  Shape and P come from the cache.
 *
 * q                [in]  device [B, H, Nq, D]
 * k_list, v_list   [in]  host arrays of P device pointers, [B, H, nk_list[p], D];
 *                        entries of reused partitions are not read (may be NULL)
 * nk_list          [in]  host array of P key counts (>= 1 where computed)
 * reuse_mask       [in]  host array of P bytes (0 fresh, 1 reuse; other values rejected)
 * o, lse           [out] device final output and LSE; they may not overlap the
 *                        cache buffer or each other.  (They may share memory
 *                        with q or the fresh K/V here, since the merge that
 *                        writes them follows the attention on `stream`, but
 *                        not in dita_attn_step_ex with a side stream.)
 * info             [in/out, nullable] step report; its `events` members, when
 *                  non-NULL, are hipEvent_t handles recorded on `stream` at the
 *                  step start, after the fresh-attention launch and at the end.
 */
typedef struct {
  int32_t n_fresh;          /* [out] partitions computed fresh                          */
  int32_t n_reused;         /* [out] partitions reused                                  */
  double fresh_flops;       /* [out] 4*B*H*Nq*sum(nk of fresh)*D                        */
  double merge_bytes;       /* [out] bytes the final merge moves: its sources and its   */
                            /*       output(s) (a group composed in the same pass too)  */
  void* ev_begin;           /* [in] hipEvent_t or NULL                                  */
  void* ev_attn_end;        /* [in] hipEvent_t or NULL                                  */
  void* ev_end;             /* [in] hipEvent_t or NULL                                  */
  int32_t merge_sources;    /* [out] states read by the final merge on `stream`         */
  int32_t premerge_sources; /* [out] reused states pre-merged on the side stream, or 0  */
  double premerge_bytes;    /* [out] (premerge_sources + 1) * bytes of one state, or 0  */
  int32_t fetched;          /* [out] reused states copied back from host memory         */
  int32_t composed;         /* [out] groups composed ahead (dita_attn_step_ex's         */
                            /*       compose_next), else 0                              */
} dita_step_info;

int dita_attn_step(dita_state_cache* cache, const void* q, const void* const* k_list,
                   const void* const* v_list, const int64_t* nk_list, const uint8_t* reuse_mask,
                   int64_t step, void* o, float* lse, void* stream, dita_step_info* info);

/*
 * dita_attn_step_ex -- dita_attn_step with the reused states composed off the
 * critical path.  Page section: State-Centric Parallel Runtime > Pipeline
 * Orchestration (reuse operations fill the bubbles of the compute pipeline).
 *
 * Reused states that were moved to host memory are copied back first (on the
 * side stream when one is given, so the copies overlap the fresh attention).
 * When opts->side_stream is non-NULL and differs from `stream`, at least one
 * partition is fresh and at least max(2, opts->min_premerge) group states are
 * reused, the reused states are merged into (o, lse) on the side stream while
 * the fresh attention runs on `stream`; the final merge on `stream` then reads
 * (o, lse) and the fresh states only and writes (o, lse) in place.  The two
 * streams are ordered by events the handle owns (created on first use, with
 * timing disabled, destroyed by dita_state_cache_free): the side stream waits
 * for all work enqueued on `stream` before the step, and `stream` waits for
 * the pre-merge before its final merge, so on return every effect is ordered
 * on `stream` as in dita_attn_step.  The result equals dita_attn_step's up to
 * the order of the fp32 sums.  opts == NULL, or no pre-merge taken, is exactly
 * dita_attn_step.  With a side stream given (non-NULL and not `stream`), o and
 * lse may not overlap q or the K/V of any partition computed fresh, since the
 * side stream may write them while the attention reads those: DITA_ERR_ARG,
 * before anything is enqueued.
 *
 * Composition ahead (opts->compose_next, the next step's reuse mask; values
 * other than 0/1: DITA_ERR_ARG before anything is enqueued).  Page section:
 * State-Centric Parallel Runtime > Dynamic Group Compose.  After this step
 * every partition holds a valid state, and the runs of partitions that
 * compose_next marks reused are composed into group states exactly as
 * dita_state_cache_compose_runs would compose them right after the step; the
 * output is the same (the final merge reads the members, not the group).
 * The run with the most groups is composed by the final merge itself in the
 * same pass over the states (its group state comes from the loads of the
 * output's merge: one pass instead of two over those states); any other run,
 * and every run when a pre-merge is taken, by a merge of its own after the
 * final one.  A run whose group state needs a free slot that a pooled cache
 * lacks is left uncomposed (info->composed counts the runs composed).  The
 * group state equals dita_state_cache_compose_runs' bit for bit when the run's
 * first partition holds a full device slot (its state is then merged first in
 * both), else up to the order of the fp32 sums.
 */
typedef struct {
  void* side_stream;     /* hipStream_t for the pre-merge, or NULL                  */
  int32_t min_premerge;  /* pre-merge only with at least this many reused states   */
  int32_t reserved;      /* must be 0                                              */
  const uint8_t* compose_next; /* host [P] reuse mask of the next step, or NULL     */
} dita_step_opts;

int dita_attn_step_ex(dita_state_cache* cache, const void* q, const void* const* k_list,
                      const void* const* v_list, const int64_t* nk_list, const uint8_t* reuse_mask,
                      int64_t step, void* o, float* lse, void* stream, const dita_step_opts* opts,
                      dita_step_info* info);

/*
 * Planner statistics.  Page section: 1. Anchor-Guided Selection Planner --
 * Error Modeling (partition importance w), Anchor Steps (w refreshed on
 * anchors) and Online Prediction (the change of the always-computed local
 * state stands in for the remote ones).
 *
 * dita_state_contrib: w_out[p] = mean over the B*H*Nq rows of
 *   exp(lse_list[p] - lse), the share of partition p in the merged softmax
 *   (rows where either LSE is -inf count 0).  lse_list: host array of P device
 *   pointers [B, H, Nq] float32; lse: the merged LSE; w_out: device, P
 *   doubles.  fp64 accumulation in a fixed order (deterministic).
 * dita_state_cache_contrib: the same over the cache's P slots (every slot must
 *   hold its own state -- no composed groups -- else DITA_ERR_STATE), with
 *   `lse` the LSE the step merged them into.
 * dita_state_change: out[0] = sum (o_new - o_prev)^2, out[1] = sum o_prev^2,
 *   out[2] = sqrt(out[0] / out[1]) (0 when both sums are 0, +inf when only
 *   out[1] is) over all B*H*Nq*D elements, fp64, summed in an order fixed by
 *   the state's size alone: the result is the same bit for bit on every run.
 *   roll != 0 also copies (o_new, lse_new) over (o_prev, lse_prev) in the same
 *   pass.  out: device, 3 doubles.  o_new/o_prev: device [B, H, Nq, D] dtype;
 *   lse_new/lse_prev: device [B, H, Nq] float32 (read/written only when
 *   rolling; may be NULL otherwise).  The new and previous buffers must not
 *   overlap.  The per-workgroup partial sums (at most 16 KB) live in scratch
 *   taken from HIP's stream-ordered allocator (hipMallocAsync on `stream`)
 *   and returned to it (hipFreeAsync) within the call.
 */
int dita_state_contrib(const dita_shape* shape, int P, const float* const* lse_list,
                       const float* lse, double* w_out, void* stream);
int dita_state_cache_contrib(const dita_state_cache* cache, const float* lse, double* w_out,
                             void* stream);
int dita_state_change(const dita_shape* shape, const void* o_new, const float* lse_new,
                      void* o_prev, float* lse_prev, int roll, double* out, void* stream);

/*
 * dita_state_change_noalloc -- dita_state_change for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, same kernels, same
 * result bit for bit; no hipMalloc, hipMallocAsync or hipFree.  The partial
 * sums live in a 16 KB array in the library's own device memory (one copy per
 * GPU, kept until the process ends; its address is looked up once per device
 * with hipGetSymbolAddress).  That array covers every state size (the grid is
 * capped at 1024 workgroups); DITA_ERR_SIZE would mean a grid beyond it.  All
 * calls on one GPU share the array and nothing in it needs clearing (each
 * call writes every partial it reads), so calls that overlap on one GPU --
 * on different streams, or from different threads without ordering -- race
 * and may return wrong sums: serialise them.
 */
int dita_state_change_noalloc(const dita_shape* shape, const void* o_new, const float* lse_new,
                              void* o_prev, float* lse_prev, int roll, double* out, void* stream);

/*
 * Error-guided planner (host only, float64).  Page section: 1. Anchor-Guided
 * Selection Planner (Error Modeling, Anchor Steps, Online Prediction,
 * Group-wise Strategy).  The page prints no formula; this one is:
 *   err_p = w_p * sum over t in (stamp_p, step] of delta~_t, where delta~_t
 *           is the change observed at the latest step <= min(t, step - 1), or
 *           the earliest observed change when none precedes t;
 *   groups = contiguous blocks of group_size partitions; a group's error is
 *           the sum over its members other than the local partition;
 *   the groups are taken in increasing (error, group index) order and reused
 *   while the running sum stays <= budget; the others are computed fresh.
 * All partitions are fresh on an anchor step (anchor_period > 0 and
 * step % anchor_period == 0), before weights are set, and before a change
 * observed at a step < `step` exists; the local partition is always fresh; a
 * group with an invalid slot is fresh, and so is (fresh_weight > 0) a group
 * holding a partition whose weight is >= fresh_weight (the page: high-
 * contribution partitions are computed).  Sums run in ascending index order.
 */
typedef struct {
  int32_t P;              /* partitions, 1..DITA_MAX_PARTITIONS                */
  int32_t q;              /* the local partition                               */
  int32_t group_size;     /* partitions per group, >= 1                        */
  int32_t anchor_period;  /* > 0: every anchor_period-th step is all fresh     */
  double budget;          /* total estimated error allowed to be reused, >= 0  */
  double fresh_weight;    /* > 0: groups with a weight >= this are always fresh */
} dita_error_plan;

typedef struct dita_planner dita_planner;

int dita_planner_create(dita_planner** out, const dita_error_plan* plan);
int dita_planner_free(dita_planner* planner);
/* w: host array of P finite, non-negative weights (e.g. from dita_state_contrib). */
int dita_planner_set_weights(dita_planner* planner, const double* w);
/* The local state's change measured at `step` (finite, >= 0); replaces an earlier value. */
int dita_planner_observe(dita_planner* planner, int64_t step, double change);
/* valid, stamp: host arrays of P entries (stamp <= step where valid); reuse_out: P
 * bytes (1 = reuse); err_out: P doubles or NULL. */
int dita_planner_mask(const dita_planner* planner, int64_t step, const uint8_t* valid,
                      const int64_t* stamp, uint8_t* reuse_out, double* err_out);
/* The same with valid/stamp read from the cache (a group member carries its group's stamp). */
int dita_planner_mask_cache(const dita_planner* planner, const dita_state_cache* cache,
                            int64_t step, uint8_t* reuse_out, double* err_out);

/*
 * Timing helpers (thin wrappers over HIP events, for benchmarks that time the
 * kernels on the stream they run on).
 */
int dita_event_create(void** event);
int dita_event_destroy(void* event);
int dita_event_record(void* event, void* stream);
/* Milliseconds between two recorded events; blocks until `stop` completes. */
int dita_event_elapsed_ms(void* start, void* stop, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* DITA_H */
