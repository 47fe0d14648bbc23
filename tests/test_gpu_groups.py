"""GPU parity of group composition and of the pre-merged (two-stream) rank-step.

Group composition (the DiTango page, State-Centric Parallel Runtime > Dynamic
Group Compose) and the step's whole-group reuse rule are checked against the
fp64 oracle's ``StateCache.compose`` / ``attn_step``: composed slot states,
group ranges, stamps, effective masks, fresh slots and merged outputs, over
multi-step schedules with drifting K/V.  The two-stream step (Pipeline
Orchestration on the same page) is checked against the oracle and against the
one-stream step on the same inputs.
"""

import numpy as np
import pytest

from gpu_util import assert_state_close, say, to_dev, to_host
from oracle import StateCache as OracleCache
from oracle import attn_step as oracle_step
from oracle import compose_runs, effective_reuse, full_attention
from workloads import round_bf16

pytestmark = pytest.mark.gpu


def _inputs(rng, H, nq, lengths, D, dtype, scale=1.2):
    # |O| stays below 2, where one bf16 rounding of the output costs at most 2^-8
    q = rng.standard_normal((1, H, nq, D)) * scale
    ks = [rng.standard_normal((1, H, n, D)) * scale for n in lengths]
    vs = [rng.standard_normal((1, H, n, D)) * 0.5 for n in lengths]
    if dtype == "bf16":
        q = round_bf16(q)
        ks = [round_bf16(x) for x in ks]
        vs = [round_bf16(x) for x in vs]
    return q, ks, vs


def _drift(rng, xs, dtype, amount=0.2):
    # variance-preserving drift: the value scale (and so bf16 rounding) stays put over steps
    keep = np.sqrt(1.0 - amount * amount)
    out = [keep * x + amount * np.std(x) * rng.standard_normal(x.shape) for x in xs]
    return [round_bf16(x) for x in out] if dtype == "bf16" else out


def _torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _check_metadata(cache, ref):
    for p in range(ref.P):
        assert cache.group(p) == ref.group_range(p), (p, cache.group(p), ref.group_range(p))
        valid, stamp = cache.info(p)
        assert (int(valid), stamp) == (int(ref.valid[p]), int(ref.stamp[p])), p
    assert cache.live() == ref.live_states()


def _check_leaders(cache, ref, dtype, what):
    for p in ref.leaders():
        if not ref.valid[p]:
            continue
        o, lse = cache.slot(p)
        ro, rl = ref.slots[p]
        assert_state_close(to_host(o), to_host(lse), ro, rl, dtype, f"{what} slot {p}")


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_compose_matches_oracle(dev, dtype, D):
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(10)
    lengths = [130, 77, 256, 190, 64, 300]
    P = len(lengths)
    q, ks, vs = _inputs(rng, 3, 200, lengths, D, dtype)
    say(f"[compose {dtype} D={D}] fill")
    cache = dita.StateCache(1, 3, 200, D, _torch_dtype(dtype), P, device=dev)
    ref = OracleCache(P)
    qd = to_dev(q, dtype, dev)
    kd = [to_dev(x, dtype, dev) for x in ks]
    vd = [to_dev(x, dtype, dev) for x in vs]
    zeros = np.zeros(P, np.uint8)
    dita.dita_attn_step(cache, qd, kd, vd, zeros, 3)
    oracle_step(ref, q, ks, vs, zeros, 3)
    # a later partial refresh so that the group stamps differ
    m = np.array([1, 1, 0, 1, 0, 1], np.uint8)
    dita.dita_attn_step(cache, qd, kd, vd, m, 5)
    oracle_step(ref, q, ks, vs, m, 5)
    # recursive composition: [1,2], then [3,4], then [1,4] (two groups), then [0,5]
    for first, last in [(1, 2), (3, 4), (1, 4)]:
        cache.compose(first, last)
        ref.compose(first, last)
        _check_metadata(cache, ref)
        _check_leaders(cache, ref, dtype, f"after compose({first},{last})")
    o_ref, lse_ref = full_attention(q, ks[1:5], vs[1:5])
    o1, l1 = cache.slot(1)
    assert_state_close(to_host(o1), to_host(l1), o_ref, lse_ref, dtype, "group [1,4] vs attention")
    cache.compose(0, 5)
    ref.compose(0, 5)
    _check_metadata(cache, ref)
    o_ref, lse_ref = full_attention(q, ks, vs)
    o0, l0 = cache.slot(0)
    assert_state_close(to_host(o0), to_host(l0), o_ref, lse_ref, dtype, "group [0,5] vs attention")
    assert cache.live() == 1 and cache.info(3) == (True, 3)
    # composing a range that already is one group changes nothing and launches nothing
    before = to_host(o0).copy()
    cache.compose(0, 5)
    assert np.array_equal(to_host(cache.slot(0)[0]), before)


def test_group_rules_on_store_load_invalidate(dev):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(11)
    P, D = 4, 64
    q, ks, vs = _inputs(rng, 2, 96, [64] * P, D, "bf16")
    cache = dita.StateCache(1, 2, 96, D, torch.bfloat16, P, device=dev)
    qd = to_dev(q, "bf16", dev)
    kd = [to_dev(x, "bf16", dev) for x in ks]
    vd = [to_dev(x, "bf16", dev) for x in vs]
    dita.dita_attn_step(cache, qd, kd, vd, np.zeros(P, np.uint8), 0)
    cache.compose(1, 3)
    so, sl = dita.dita_attn_partial(qd, kd[0], vd[0])
    for p in (1, 2, 3):
        with pytest.raises(dita.DitaError) as e:
            cache.store(p, so, sl, 1)
        assert e.value.status == dita.DITA_ERR_STATE
    for p in (2, 3):
        with pytest.raises(dita.DitaError) as e:
            cache.load(p)
        assert e.value.status == dita.DITA_ERR_STATE
    lo, ll = cache.load(1)
    o_ref, lse_ref = full_attention(q, ks[1:], vs[1:])
    assert_state_close(to_host(lo), to_host(ll), o_ref, lse_ref, "bf16", "load of a group leader")
    with pytest.raises(dita.DitaError):
        cache.compose(2, 3)             # straddles the group [1, 3]
    with pytest.raises(dita.DitaError):
        cache.compose(0, 2)
    cache.invalidate(2)                 # the whole group goes
    assert [cache.info(p)[0] for p in range(P)] == [True, False, False, False]
    assert [cache.group(p) for p in range(P)] == [(0, 0), (1, 1), (2, 2), (3, 3)]
    cache.store(2, so, sl, 7)           # a single slot again
    assert cache.info(2) == (True, 7)


# Schedules over 6 partitions: (mask, composition applied after the step).
SCHEDULE = [
    ([0, 0, 0, 0, 0, 0], [(2, 3), (4, 5)]),
    ([0, 1, 1, 1, 1, 1], [(2, 5)]),
    ([0, 0, 1, 1, 1, 1], []),
    ([0, 1, 1, 0, 1, 1], [(1, 2)]),      # partition 3 fresh: group [2,5] recomputed whole
    ([0, 1, 1, 1, 1, 1], [(3, 5), (0, 2)]),
    ([1, 1, 1, 1, 0, 1], []),            # group [3,5] recomputed; group [0,2] reused
    ([0, 1, 1, 1, 1, 1], []),
]


def _compose_ahead_schedule(n_steps, P, seed):
    """Masks of a random schedule (local partition 0 always fresh, anchors every
    5th step); after each step the next step's reuse runs are composed."""
    rng = np.random.default_rng(seed)
    masks = []
    for s in range(n_steps):
        m = (rng.random(P) < 0.6).astype(np.uint8)
        m[0] = 0
        if s % 5 == 0:
            m[:] = 0
        masks.append(m)
    return [(list(masks[s]), masks[s + 1] if s + 1 < n_steps else None) for s in range(n_steps)]


def _run_schedule(dev, dtype, D, side, schedule=None):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(12)
    lengths = [200, 129, 256, 70, 333, 190]
    P, H, nq = len(lengths), 3, 230
    q, ks, vs = _inputs(rng, H, nq, lengths, D, dtype)
    cache = dita.StateCache(1, H, nq, D, _torch_dtype(dtype), P, device=dev)
    ref = OracleCache(P)
    qd = to_dev(q, dtype, dev)
    stream = torch.cuda.Stream(device=dev) if side else None
    o = torch.empty((1, H, nq, D), dtype=_torch_dtype(dtype), device=dev)
    lse = torch.empty((1, H, nq), dtype=torch.float32, device=dev)
    outs = []
    for s, (mask, comps) in enumerate(SCHEDULE if schedule is None else schedule):
        mask = np.array(mask, np.uint8)
        eff = effective_reuse(ref, mask)
        assert np.array_equal(cache.effective_mask(mask), eff), (s, cache.effective_mask(mask), eff)
        kd = [to_dev(x, dtype, dev) for x in ks]
        vd = [to_dev(x, dtype, dev) for x in vs]
        live_reused = sum(1 for p in ref.leaders() if eff[p])
        # the same output buffers every step: the side stream must not overtake their readers
        _, _, info = dita.dita_attn_step(cache, qd, kd, vd, mask, s, o=o, lse=lse, side_stream=stream)
        o_ref, lse_ref, nf = oracle_step(ref, q, ks, vs, mask, s)
        assert info.n_fresh == nf == int((eff == 0).sum())
        pre = side and nf > 0 and live_reused >= 2
        assert info.premerge_sources == (live_reused if pre else 0), (s, info.premerge_sources)
        assert info.merge_sources == (1 + nf if pre else len(ref.leaders())), s
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, f"step {s} output")
        outs.append((to_host(o).copy(), to_host(lse).copy()))
        for p in np.flatnonzero(eff == 0):
            so, sl = cache.slot(int(p))
            ro, rl = ref.slots[p]
            assert_state_close(to_host(so), to_host(sl), ro, rl, dtype, f"step {s} fresh slot {p}")
        if isinstance(comps, np.ndarray):       # compose the next step's reuse runs
            assert cache.compose_runs(comps) == compose_runs(ref, comps)
        elif comps is not None:
            for first, last in comps:
                cache.compose(first, last)
                ref.compose(first, last)
        _check_metadata(cache, ref)
        _check_leaders(cache, ref, dtype, f"step {s}")
        ks = _drift(rng, ks, dtype)
        vs = _drift(rng, vs, dtype)
    return outs


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_group_schedule_matches_oracle(dev, dtype, D):
    say(f"[group schedule {dtype} D={D}] one stream")
    _run_schedule(dev, dtype, D, side=False)


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 128), ("bf16", 64)])
def test_premerge_schedule_matches_oracle_and_one_stream(dev, dtype, D):
    say(f"[premerge schedule {dtype} D={D}] two streams vs one")
    a = _run_schedule(dev, dtype, D, side=True)
    b = _run_schedule(dev, dtype, D, side=False)
    for s, ((oa, la), (ob, lb)) in enumerate(zip(a, b)):
        # same states, merged in a different order of fp32 sums
        assert_state_close(oa, la, ob, lb, dtype, f"step {s} two-stream vs one-stream")


@pytest.mark.parametrize("side", [False, True])
def test_compose_ahead_schedule_matches_oracle(dev, side):
    say(f"[compose-ahead schedule side={side}]")
    _run_schedule(dev, "bf16", 128, side, schedule=_compose_ahead_schedule(12, 6, seed=3))


@pytest.mark.parametrize("pooled", [False, True])
def test_step_composes_ahead_like_compose_runs(dev, pooled):
    """dita_attn_step_ex with compose_next: the step composes the next step's
    reused runs itself, the largest one in the same pass as its final merge.
    Against the plain step followed by compose_runs on a second cache, over a
    schedule with two runs per reuse step (one fused into the merge, one merged
    on its own) and an all-fresh step in between: outputs, group ranges and
    group states bit for bit (the runs start at partitions that hold full
    slots), and the count of composed runs."""
    import torch
    import partial_state_reuse_amd as dita
    H, nq, D, P, n = 4, 300, 128, 8, 260
    rng = np.random.default_rng(11 + pooled)
    q, ks, vs = _inputs(rng, H, nq, [n] * P, D, "bf16")
    tq = to_dev(q, "bf16", dev)
    fresh = np.zeros(P, np.uint8)
    near = np.array([1, 1, 0, 0, 0, 1, 1, 1], np.uint8)  # runs [0, 1] and [5, 7]
    masks = [fresh, near, near, fresh, near, near]
    slots = P if pooled else None
    a = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=slots)
    b = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=slots)
    for s, mask in enumerate(masks):
        nxt = masks[s + 1] if s + 1 < len(masks) else None
        tk = [to_dev(x, "bf16", dev) for x in ks]
        tv = [to_dev(x, "bf16", dev) for x in vs]
        oa, la, ia = dita.dita_attn_step(a, tq, tk, tv, mask, s, compose_next=nxt)
        ob, lb, _ = dita.dita_attn_step(b, tq, tk, tv, mask, s)
        runs = b.compose_runs(nxt) if nxt is not None else 0
        torch.cuda.synchronize()
        say(f"  step {s} pooled={pooled}: composed {ia.composed}, compose_runs launched {runs}")
        assert np.array_equal(to_host(oa), to_host(ob)) and np.array_equal(to_host(la), to_host(lb)), s
        assert ia.composed == (2 if nxt is not None and (mask == 0).all() else 0), (s, ia.composed)
        for p in range(P):
            assert a.group(p) == b.group(p), (s, p, a.group(p), b.group(p))
            assert a.info(p) == b.info(p), (s, p)
        for p in range(P):
            if a.group(p)[0] != p:
                continue
            so, sl = a.slot(p)
            ro, rl = b.slot(p)
            assert np.array_equal(to_host(so), to_host(ro)) and np.array_equal(to_host(sl), to_host(rl)), (s, p)
        ks = _drift(rng, ks, "bf16")
        vs = _drift(rng, vs, "bf16")


def test_step_composes_ahead_with_premerge(dev):
    """compose_next together with the side-stream pre-merge: on steps that
    pre-merge their reused states the runs are composed by merges of their own
    after the final merge, on all-fresh steps by the final merge itself.
    Against the same two-stream step followed by compose_runs: outputs, group
    ranges and group states bit for bit, and the count of composed runs."""
    import torch
    import partial_state_reuse_amd as dita
    H, nq, D, P, n = 4, 300, 128, 8, 260
    rng = np.random.default_rng(23)
    q, ks, vs = _inputs(rng, H, nq, [n] * P, D, "bf16")
    tq = to_dev(q, "bf16", dev)
    fresh = np.zeros(P, np.uint8)
    m_a = np.array([1, 1, 0, 0, 0, 0, 1, 0], np.uint8)  # reused: group [0, 1] and 6
    m_b = np.array([1, 1, 0, 0, 0, 1, 1, 1], np.uint8)  # then also 5 and 7: run [5, 7]
    masks = [fresh, m_a, m_b, fresh, m_a, m_b]
    want = [1, 1, 0, 1, 1, 0]  # runs composed: [0, 1]; [5, 7]; none; ...
    side = torch.cuda.Stream(device=dev)
    a = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    b = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    for s, mask in enumerate(masks):
        nxt = masks[s + 1] if s + 1 < len(masks) else None
        tk = [to_dev(x, "bf16", dev) for x in ks]
        tv = [to_dev(x, "bf16", dev) for x in vs]
        oa, la, ia = dita.dita_attn_step(a, tq, tk, tv, mask, s, side_stream=side, compose_next=nxt)
        ob, lb, ib = dita.dita_attn_step(b, tq, tk, tv, mask, s, side_stream=side)
        if nxt is not None:
            b.compose_runs(nxt)
        torch.cuda.synchronize()
        say(f"  step {s}: premerged {ia.premerge_sources}, composed {ia.composed}")
        assert ia.premerge_sources == ib.premerge_sources, s
        assert np.array_equal(to_host(oa), to_host(ob)) and np.array_equal(to_host(la), to_host(lb)), s
        assert ia.composed == want[s], (s, ia.composed)
        for p in range(P):
            assert a.group(p) == b.group(p), (s, p, a.group(p), b.group(p))
            assert a.info(p) == b.info(p), (s, p)
            if a.group(p)[0] == p:
                so, sl = a.slot(p)
                ro, rl = b.slot(p)
                assert np.array_equal(to_host(so), to_host(ro)) and np.array_equal(to_host(sl), to_host(rl)), (s, p)
        ks = _drift(rng, ks, "bf16")
        vs = _drift(rng, vs, "bf16")
