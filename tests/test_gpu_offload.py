"""GPU tests of host offload and of the pooled cache.

States moved to pinned host memory and copied back (explicitly, or by a step
that reuses them, on the step's stream or on a side stream overlapping the
fresh attention) must come back bit for bit: a step over offloaded states must
return exactly what the same step over resident states returns.  A pooled
cache (fewer physical slots than partitions) filled in chunks and composed as
it goes must match the fp64 oracle, keep within its slots, and refuse a step
that needs more slots before launching anything.
"""

import numpy as np
import pytest

from gpu_util import assert_state_close, say, to_dev, to_host
from oracle import StateCache as OracleCache
from oracle import attn_step as oracle_step
from oracle import partial_state
from workloads import round_bf16

pytestmark = pytest.mark.gpu


def _inputs(rng, H, nq, lengths, D):
    q = round_bf16(rng.standard_normal((1, H, nq, D)) * 1.2)
    ks = [round_bf16(rng.standard_normal((1, H, n, D)) * 1.2) for n in lengths]
    vs = [round_bf16(rng.standard_normal((1, H, n, D)) * 0.5) for n in lengths]
    return q, ks, vs


def _dev(xs, dev):
    return [to_dev(x, "bf16", dev) for x in xs]


def _same(a, b):
    return bool((a == b).all())


def test_offload_fetch_roundtrip_bitwise(dev):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(30)
    P, H, nq, D = 4, 3, 300, 128
    q, ks, vs = _inputs(rng, H, nq, [200, 150, 260, 90], D)
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    qd, kd, vd = to_dev(q, "bf16", dev), _dev(ks, dev), _dev(vs, dev)
    dita.dita_attn_step(cache, qd, kd, vd, np.zeros(P, np.uint8), 0)
    before = [tuple(x.clone() for x in cache.slot(p)) for p in range(P)]
    cache.offload(2)
    assert cache.residency() == (3, 1, 1)
    lo, ll = cache.load(2)                       # served from the host copy
    torch.cuda.synchronize()
    assert _same(lo, before[2][0]) and _same(ll, before[2][1])
    with pytest.raises(dita.DitaError) as e:
        cache.offload(2)                         # already on the host
    assert e.value.status == dita.DITA_ERR_STATE
    cache.slot(2)[0].zero_()                     # the device copy is no longer the state
    cache.fetch(2)
    torch.cuda.synchronize()
    assert _same(cache.slot(2)[0], before[2][0]) and _same(cache.slot(2)[1], before[2][1])
    assert cache.residency() == (4, 0, 0)


@pytest.mark.parametrize("mode,D", [("stream", 128), ("side", 128), ("side_premerge", 128),
                                    ("side", 64)])
def test_step_fetches_offloaded_states(dev, mode, D):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(31)
    lengths = [200, 129, 256, 70, 333, 190]
    P, H, nq = len(lengths), 3, 230
    q, ks, vs = _inputs(rng, H, nq, lengths, D)
    qd, kd, vd = to_dev(q, "bf16", dev), _dev(ks, dev), _dev(vs, dev)
    _, ks1, vs1 = _inputs(np.random.default_rng(32), H, nq, lengths, D)
    kd1, vd1 = _dev(ks1, dev), _dev(vs1, dev)
    side = torch.cuda.Stream(device=dev) if mode != "stream" else None
    min_pre = 0 if mode == "side_premerge" else 64
    outs = []
    for offload in (False, True):
        cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
        ref = OracleCache(P)
        dita.dita_attn_step(cache, qd, kd, vd, np.zeros(P, np.uint8), 0)
        oracle_step(ref, q, ks, vs, np.zeros(P, np.uint8), 0)
        cache.compose(3, 5)
        ref.compose(3, 5)
        if offload:
            cache.offload(3)
            cache.offload(2)
            assert cache.residency() == (2, 2, 4)
        mask = np.array([0, 0, 1, 1, 1, 1], np.uint8)
        o, lse, info = dita.dita_attn_step(cache, qd, kd1, vd1, mask, 1, side_stream=side,
                                           min_premerge=min_pre)
        o_ref, lse_ref, _ = oracle_step(ref, q, ks1, vs1, mask, 1)
        assert info.fetched == (2 if offload else 0)
        assert cache.residency() == (4, 0, 2)
        torch.cuda.synchronize()
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", f"{mode} offload={offload}")
        outs.append((o.clone(), lse.clone()))
    if mode != "side_premerge":
        # the same sources in the same order: bit for bit
        assert _same(outs[0][0], outs[1][0]) and _same(outs[0][1], outs[1][1])


def test_pooled_cache_chunked_fill_and_steps(dev):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(33)
    lengths = [180, 160, 240, 120, 300, 200]
    P, S, H, nq, D = len(lengths), 3, 3, 210, 64
    q, ks, vs = _inputs(rng, H, nq, lengths, D)
    qd, kd, vd = to_dev(q, "bf16", dev), _dev(ks, dev), _dev(vs, dev)
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=S)
    assert cache.buffer.numel() == dita.lib().dita_state_cache_bytes(ctypes_shape(cache), S)
    ref = OracleCache(P)
    # chunked cold fill: each new partition is stored, then folded into the far group
    for p in range(P):
        say(f"[pool] store {p}")
        o, l = dita.dita_attn_partial(qd, kd[p], vd[p])
        cache.store(p, o, l, 0)
        ref.store(p, partial_state(q, ks[p], vs[p]), 0)
        if p >= 2:
            cache.compose(1, p)
            ref.compose(1, p)
        assert cache.residency()[0] <= S
    assert cache.residency() == (2, 0, 1) and cache.group(4) == (1, 5)
    mask = np.array([0, 1, 1, 1, 1, 1], np.uint8)
    o1, l1, info = dita.dita_attn_step(cache, qd, kd, vd, mask, 1)
    o_ref, lse_ref, nf = oracle_step(ref, q, ks, vs, mask, 1)
    assert info.n_fresh == nf == 1
    assert_state_close(to_host(o1), to_host(l1), o_ref, lse_ref, "bf16", "pooled step")
    first = (o1.clone(), l1.clone())
    # move the group to the host: one slot in use; the next step brings it back
    cache.offload(1)
    assert cache.residency() == (1, 1, 2)
    o2, l2, info = dita.dita_attn_step(cache, qd, kd, vd, mask, 2)
    assert info.fetched == 1 and cache.residency() == (2, 0, 1)
    torch.cuda.synchronize()
    assert _same(o2, first[0]) and _same(l2, first[1])
    # recomputing the group needs six slots: refused before any launch, nothing changes
    with pytest.raises(dita.DitaError) as e:
        dita.dita_attn_step(cache, qd, kd, vd, np.array([0, 0, 1, 1, 1, 1], np.uint8), 3)
    assert e.value.status == dita.DITA_ERR_SIZE
    assert cache.residency() == (2, 0, 1) and cache.group(3) == (1, 5)
    o3, l3, _ = dita.dita_attn_step(cache, qd, kd, vd, mask, 3)
    torch.cuda.synchronize()
    assert _same(o3, first[0])


def ctypes_shape(cache):
    import ctypes
    return ctypes.byref(cache.shape)


def test_everything_together_matches_oracle(dev):
    """Random masks, composition ahead of each step, random moves of group states to
    the host, a pooled cache and a side stream with pre-merge, over 14 steps with
    drifting K/V: every output against the fp64 oracle."""
    import torch
    import partial_state_reuse_amd as dita
    from oracle import compose_runs as oracle_compose_runs
    rng = np.random.default_rng(34)
    lengths = [150, 96, 210, 64, 180, 120, 240, 77]
    P, H, nq, D = len(lengths), 2, 190, 128
    q, ks, vs = _inputs(rng, H, nq, lengths, D)
    qd = to_dev(q, "bf16", dev)
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=P)
    ref = OracleCache(P)
    side = torch.cuda.Stream(device=dev)
    masks = []
    for s in range(14):
        m = (rng.random(P) < 0.65).astype(np.uint8)
        m[0] = 0
        if s % 6 == 0:
            m[:] = 0
        masks.append(m)
    for s, m in enumerate(masks):
        kd, vd = _dev(ks, dev), _dev(vs, dev)
        o, lse, info = dita.dita_attn_step(cache, qd, kd, vd, m, s, side_stream=side)
        o_ref, lse_ref, nf = oracle_step(ref, q, ks, vs, m, s)
        assert info.n_fresh == nf
        torch.cuda.synchronize()
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", f"step {s}")
        if s + 1 < len(masks):
            assert cache.compose_runs(masks[s + 1]) == oracle_compose_runs(ref, masks[s + 1])
            for p in ref.leaders():
                if ref.group_range(p)[1] > p and rng.random() < 0.5:
                    cache.offload(p)
        on_dev, on_host, free = cache.residency()
        assert on_dev + on_host == ref.live_states() and on_dev + free == P
        ks = [round_bf16(0.98 * x + 0.2 * rng.standard_normal(x.shape)) for x in ks]
        vs = [round_bf16(0.98 * x + 0.1 * rng.standard_normal(x.shape)) for x in vs]


def test_sixty_four_partitions_with_groups_and_offload(dev):
    """The largest cache (64 partitions, pooled): a growing near set recomputed, with
    composition ahead of each step and the far groups moved to the host, against
    the oracle."""
    import torch
    import partial_state_reuse_amd as dita
    from oracle import compose_runs as oracle_compose_runs
    rng = np.random.default_rng(35)
    P, H, nq, D = 64, 2, 96, 64
    lengths = [int(x) for x in rng.integers(16, 80, P)]
    q, ks, vs = _inputs(rng, H, nq, lengths, D)
    qd, kd, vd = to_dev(q, "bf16", dev), _dev(ks, dev), _dev(vs, dev)
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=P)
    ref = OracleCache(P)
    masks = [np.zeros(P, np.uint8)]
    for s in range(1, 6):
        m = np.ones(P, np.uint8)
        m[: 2 + s] = 0                                  # a growing near set recomputed
        masks.append(m)
    side = torch.cuda.Stream(device=dev)
    for s, m in enumerate(masks):
        o, lse, info = dita.dita_attn_step(cache, qd, kd, vd, m, s, side_stream=side)
        o_ref, lse_ref, nf = oracle_step(ref, q, ks, vs, m, s)
        assert info.n_fresh == nf
        torch.cuda.synchronize()
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", f"P=64 step {s}")
        if s + 1 < len(masks):
            cache.compose_runs(masks[s + 1])
            oracle_compose_runs(ref, masks[s + 1])
            for p in ref.leaders():
                if ref.group_range(p)[1] > p:
                    cache.offload(p)
            assert cache.residency()[1] == sum(1 for p in ref.leaders() if ref.group_range(p)[1] > p)


def _random_state(rng, H, nq, D):
    o = round_bf16(rng.standard_normal((1, H, nq, D)) * 0.7)
    lse = (rng.standard_normal((1, H, nq)) + 6.0).astype(np.float32)
    return o, lse


def test_pooled_slot_released_on_one_stream_taken_on_another(dev):
    """Offload on stream A frees a pooled slot; a step on stream B fetches the state
    back into that slot and reuses the other, which A stored.  Stream A is held
    back first by a bounded sleep kernel, so B's work would run ahead of A's
    copies if the library did not order the slots: the result must still be the
    oracle's merge of the two stored states, and the host copy exact."""
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(36)
    H, nq, D, P = 16, 2048, 128, 2
    x0, x1 = _random_state(rng, H, nq, D), _random_state(rng, H, nq, D)
    a, b = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=2)
    d0 = (to_dev(x0[0], "bf16", dev), torch.from_numpy(x0[1]).to(dev))
    d1 = (to_dev(x1[0], "bf16", dev), torch.from_numpy(x1[1]).to(dev))
    torch.cuda.synchronize()
    with torch.cuda.stream(a):
        torch.cuda._sleep(20_000_000)               # ~10 ms, bounded
    cache.store(0, *d0, step=0, stream=a)
    cache.store(1, *d1, step=0, stream=a)
    ho, hl = cache.offload(1, stream=a)
    assert cache.residency() == (1, 1, 1)
    q = to_dev(np.zeros((1, H, nq, D), np.float32), "bf16", dev)
    o, lse, info = dita.dita_attn_step(cache, q, [None, None], [None, None],
                                       np.ones(P, np.uint8), 1, stream=b)
    assert info.fetched == 1
    torch.cuda.synchronize()
    assert np.array_equal(ho.float().numpy(), x1[0]) and np.array_equal(hl.numpy(), x1[1])
    ref = OracleCache(P)
    ref.store(0, x0, 0)
    ref.store(1, x1, 0)
    o_ref, lse_ref, _ = oracle_step(ref, None, [None, None], [None, None], np.ones(P, np.uint8), 1)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "two-stream pooled fetch")


def test_pooled_slot_freed_by_compose_then_written_on_another_stream(dev):
    """Composition on stream A frees a member's pooled slot; a step on stream B
    recomputes the group, so its attention writes that slot and the leader's.
    With A held back by a bounded sleep, only the library's ordering keeps B from
    writing before A's in-place merge has read and written them."""
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(37)
    H, nq, D, P = 8, 1024, 128, 3
    lengths = [300, 200, 250]
    q, ks, vs = _inputs(rng, H, nq, lengths, D)
    xs = [_random_state(rng, H, nq, D) for _ in range(P)]
    a, b = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev, slots=3)
    dx = [(to_dev(x[0], "bf16", dev), torch.from_numpy(x[1]).to(dev)) for x in xs]
    qd, kd, vd = to_dev(q, "bf16", dev), _dev(ks, dev), _dev(vs, dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(a):
        torch.cuda._sleep(20_000_000)
    for p in range(P):
        cache.store(p, *dx[p], step=0, stream=a)
    cache.compose(0, 1, stream=a)
    assert cache.residency() == (2, 0, 1)
    mask = np.array([0, 0, 1], np.uint8)
    o, lse, info = dita.dita_attn_step(cache, qd, kd, vd, mask, 1, stream=b)
    assert info.n_fresh == 2
    torch.cuda.synchronize()
    ref = OracleCache(P)
    for p in range(P):
        ref.store(p, xs[p], 0)
    ref.compose(0, 1)
    o_ref, lse_ref, _ = oracle_step(ref, q, ks, vs, mask, 1)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "two-stream pooled compose")
