"""GPU parity of compact cached states (int8 codes with a per-row scale).

The encoding is bit-exact: on identical bf16 states (seeded inputs, stored
into the cache) the library's codes, scales and LSE equal the oracle's
encoder's bit for bit, over ragged row counts, both head sizes, zero rows,
exact ties and a wide dynamic range.  Merges and compositions that read
compact states match the oracle's merge of the decoded values within the
acceptance tolerances.  A schedule that compacts the states its next step
reuses matches the oracle doing the same; the reading for that comparison is
stated at the test (the two sides encode their own bf16 states, which may
differ by one bf16 unit, so a code may differ by one step).
"""

import numpy as np
import pytest

import workloads
from gpu_util import assert_state_close, say, to_dev, to_host
from oracle import StateCache as OracleCache
from oracle import attn_step as oracle_step
from oracle import compose_runs as oracle_compose_runs
from oracle.compress import bf16_round, decode_rows, encode_rows
from workloads import Inputs, split_parts

pytestmark = pytest.mark.gpu


def _state(rng, shape, spread=True, ties=True):
    """A bf16 state with a zero row, rows of exact ties (ties=True, at magnitudes up
    to 2^17) and rows of very different magnitude (spread=True)."""
    o = rng.standard_normal(shape)
    if spread:
        o *= 10.0 ** rng.uniform(-6, 3, shape[:-1])[..., None]
    else:
        o *= 0.4        # the size of attention outputs: convex combinations of value rows
    o = bf16_round(o)
    flat = o.reshape(-1, shape[-1])
    if flat.shape[0] > 3:
        flat[3] = 0.0
    n = max(0, min(8, flat.shape[0] - 5)) if ties else 0
    for r in range(5, 5 + n):                     # rows of exact halves: a = 127 * 2^e
        e = int(rng.integers(-10, 10))
        k = rng.integers(-126, 126, shape[-1]).astype(np.float64)
        flat[r] = bf16_round((k + 0.5) * 2.0 ** e)
        flat[r, 0] = np.float32(127 * 2.0 ** e)
    lse = (rng.standard_normal(shape[:-1]) * 3 + 5).astype(np.float32)
    return o.astype(np.float32), lse


@pytest.mark.parametrize("H,nq,D", [(3, 333, 128), (2, 517, 64), (1, 1, 128)])
def test_encoding_is_bit_exact(dev, H, nq, D):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(60 + D + nq)
    P = 2
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=2, compact_slots=2)
    for p in range(P):
        o, lse = _state(rng, (1, H, nq, D), spread=(p == 0))
        cache.store(p, to_dev(o, "bf16", dev), torch.from_numpy(lse).to(dev), step=0)
        cache.compact(p)
        assert cache.format(p) == dita.DITA_STATE_COMPACT
        codes, scale, lse_c = cache.compact_slot(p)
        torch.cuda.synchronize()
        ref_codes, ref_scale = encode_rows(o)
        assert np.array_equal(codes.cpu().numpy(), ref_codes), "codes differ"
        got_s = scale.cpu().numpy()
        assert np.array_equal(got_s.view(np.uint32), ref_scale.view(np.uint32)), "scales differ"
        assert np.array_equal(lse_c.cpu().numpy().view(np.uint32), lse.view(np.uint32))
    assert cache.residency() == (2, 0, 2)        # both full slots went back to the pool


def test_merge_and_compose_read_compact_states(dev):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(61)
    P, H, nq, D = 5, 3, 300, 128
    states = [_state(rng, (1, H, nq, D), spread=False, ties=False) for _ in range(P)]
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=4, compact_slots=4)
    ref = OracleCache(P)
    for p, (o, lse) in enumerate(states):
        if p == 4:                                 # four full slots: compact before the fifth store
            for c in (1, 2, 3):
                cache.compact(c)
                ref.compact(c)
        cache.store(p, to_dev(o, "bf16", dev), torch.from_numpy(lse).to(dev), step=0)
        ref.store(p, (o.astype(np.float64), lse.astype(np.float64)), 0)
    assert [cache.format(p) for p in range(P)] == [1, 2, 2, 2, 1]
    reuse = np.ones(P, np.uint8)
    o, l, info = dita.dita_attn_step(cache, torch.zeros((1, H, nq, D), dtype=torch.bfloat16, device=dev),
                                     [None] * P, [None] * P, reuse, 1)
    o_ref, l_ref, _ = oracle_step(ref, None, [None] * P, [None] * P, reuse, 1)
    assert info.merge_sources == P
    assert_state_close(to_host(o), to_host(l), o_ref, l_ref, "bf16", "merge with compact sources")
    # compose a range of compact states only (out of place, into a free full slot)
    cache.compose(1, 2)
    ref.compose(1, 2)
    assert cache.format(1) == dita.DITA_STATE_FULL and cache.group(2) == (1, 2)
    # compose a full state with a compact group member range (in place)
    cache.compose(3, 4)
    ref.compose(3, 4)
    assert cache.format(3) == dita.DITA_STATE_FULL
    for p in (1, 3):
        so, sl = cache.slot(p)
        ro, rl = ref.slots[p]
        assert_state_close(to_host(so), to_host(sl), ro, rl, "bf16", f"group led by {p}")
    o2, l2, _ = dita.dita_attn_step(cache, torch.zeros((1, H, nq, D), dtype=torch.bfloat16, device=dev),
                                    [None] * P, [None] * P, reuse, 2)
    o2_ref, l2_ref, _ = oracle_step(ref, None, [None] * P, [None] * P, reuse, 2)
    assert_state_close(to_host(o2), to_host(l2), o2_ref, l2_ref, "bf16", "after composition")


def test_schedule_with_compaction_matches_oracle(dev):
    """The 50-step ramp schedule's shape on a smaller grid, composing ahead and then
    compacting every state the next step reuses, on both sides.

    Reading for the tolerance: each side encodes its own bf16 state, and the
    library's fp32-accumulated state may differ from the oracle's by one bf16
    unit, which can move a code by one step s = a/127 of its row.  A reused
    compact state enters the output with weight w_p = exp(LSE_p - LSE), so
    per row the outputs may differ by the bf16 tolerance plus
    sum_p w_p * 2 s_p over the compact states p (one unit for the differing
    input, one code step).  LSE is kept exactly and has the usual tolerance."""
    import torch
    import partial_state_reuse_amd as dita
    from gpu_util import TOL
    wl = workloads.reduced("dit75k_ramp50", H=4, grid=(21, 15, 16), steps=16)
    P = wl.P
    inp = Inputs(wl, seed=9)
    q_dev = to_dev(inp.q, "bf16", dev)
    cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, torch.bfloat16, P, device=dev, slots=P,
                            compact_slots=P - 1)
    ref = OracleCache(P)
    plan = dita.Plan(**wl.plan_fields())
    steps_of = {}                                  # leader -> per-row code step of its compact state
    n_compact_reused = 0
    for s in range(wl.steps):
        k, v = inp.kv(s)
        mask = dita.dita_plan_mask(plan, s, cache)
        ks = [to_dev(np.ascontiguousarray(x), "bf16", dev) for x in split_parts(k, wl)]
        vs = [to_dev(np.ascontiguousarray(x), "bf16", dev) for x in split_parts(v, wl)]
        o, lse, info = dita.dita_attn_step(cache, q_dev, ks, vs, mask, s)
        o_ref, lse_ref, nf = oracle_step(ref, inp.q, split_parts(k, wl), split_parts(v, wl), mask, s)
        assert info.n_fresh == nf
        compact_now = [p for p in ref.leaders() if p in steps_of and mask[p] == 1]
        n_compact_reused += len(compact_now)
        bound = np.zeros(lse_ref.shape)
        for p in compact_now:
            bound += np.exp(ref.slots[p][1] - lse_ref) * 2 * steps_of[p]
        tol_o, tol_l = TOL["bf16"]
        d = np.abs(to_host(o) - o_ref)
        assert np.all(d <= tol_o + bound[..., None]), f"step {s}: O beyond the stated bound"
        assert np.max(np.abs(to_host(lse) - lse_ref)) <= tol_l
        for p in np.flatnonzero(mask == 0):
            steps_of.pop(int(p), None)             # recomputed: full again
        say(f"[compact schedule] step {s}: fresh {nf}/{P}, compact reused {len(compact_now)}, "
            f"O err {d.max():.2e} (bound {tol_o + bound.max():.2e})")
        if s + 1 < wl.steps:
            nxt = dita.dita_plan_mask(plan, s + 1, cache)
            before = {p: ref.group_range(p) for p in steps_of}
            cache.compose_runs(nxt)
            oracle_compose_runs(ref, nxt)
            # a leader whose group grew was merged into a new (full) state
            steps_of = {p: v for p, v in steps_of.items()
                        if ref.group[p] == p and ref.group_range(p) == before[p]}
            for p in ref.leaders():
                if nxt[p] == 1 and cache.format(p) == dita.DITA_STATE_FULL:
                    o_p = bf16_round(ref.slots[p][0])
                    steps_of[p] = np.max(np.abs(o_p.astype(np.float64)), axis=-1) / 127
                    cache.compact(p)
                    ref.compact(p)
            assert all(cache.format(p) == dita.DITA_STATE_COMPACT for p in steps_of)
    assert n_compact_reused > 0
