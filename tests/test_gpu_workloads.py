"""GPU parity of whole rank-step schedules on the five synthetic workloads.

For every step: the library's mask must equal the oracle planner's bit for
bit; the fresh states written into the cache, and the merged output and LSE,
must match the oracle's within the acceptance tolerances.  The two small
workloads are compared in full; the video-DiT shapes run at full size on the
GPU and are compared on a fixed sample of heads and query rows that the fp64
oracle recomputes exactly (attention rows are independent, so the restricted
oracle is the full oracle on those rows).
"""

import numpy as np
import pytest

import workloads
from gpu_util import assert_state_close, say, to_dev, to_host
from oracle import Plan as OraclePlan
from oracle import StateCache as OracleCache
from oracle import attn_step as oracle_step
from oracle import compose_runs as oracle_compose_runs
from oracle import full_attention
from oracle import plan_mask as oracle_mask
from workloads import Inputs, split_parts

pytestmark = pytest.mark.gpu


def partition_tensors(x: np.ndarray, wl, dev):
    """[B, H, N, D] host array -> P contiguous [B, H, Nk, D] device tensors."""
    return [to_dev(np.ascontiguousarray(x[:, :, a:b]), wl.dtype, dev)
            for a, b in (wl.part_range(p) for p in range(wl.P))]


def sample_rows(wl):
    if wl.H * wl.Nq <= 12 * 2048:
        return None, None
    heads = sorted({0, 13, 26, 39} & set(range(wl.H)))
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(wl.Nq - 70, wl.Nq),
                                     rng.choice(wl.Nq, 64, replace=False)]))
    return heads, rows


def run_schedule(wl, dev, steps=None, seed=0, compose_ahead=False):
    """Run the workload's schedule on both sides.  With ``compose_ahead`` the
    runs of partitions the next step reuses are composed into groups after
    every step (the benchmark's default pipeline), on both sides."""
    import torch
    import partial_state_reuse_amd as dita
    steps = wl.steps if steps is None else steps
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    say(f"[{wl.name}] generating inputs H={wl.H} N={wl.N} P={wl.P}")
    inp = Inputs(wl, seed=seed)
    heads, rows = sample_rows(wl)
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads][:, :, rows])
    selk = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    q_dev = to_dev(inp.q, wl.dtype, dev)
    q_ref = sel(inp.q)
    cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev)
    ref_cache = OracleCache(wl.P)
    plan = dita.Plan(**wl.plan_fields())
    ref_plan = OraclePlan(**wl.plan_fields())
    worst = [0.0, 0.0]
    fresh_total = 0
    for s in range(steps):
        k, v = inp.kv(s)
        mask = dita.dita_plan_mask(plan, s, cache)
        ref_m = oracle_mask(ref_plan, s, ref_cache.valid)
        assert np.array_equal(mask, ref_m), (s, mask, ref_m)
        ks, vs = partition_tensors(k, wl, dev), partition_tensors(v, wl, dev)
        o, lse, info = dita.dita_attn_step(cache, q_dev, ks, vs, mask, s)
        kp = [selk(x) for x in split_parts(k, wl)]
        vp = [selk(x) for x in split_parts(v, wl)]
        o_ref, lse_ref, nf = oracle_step(ref_cache, q_ref, kp, vp, mask, s)
        assert info.n_fresh == nf == int((mask == 0).sum())
        fresh_total += nf
        eo, el = assert_state_close(sel(to_host(o)), sel(to_host(lse)), o_ref, lse_ref, wl.dtype,
                                    f"{wl.name} step {s} output")
        for p in np.flatnonzero(mask == 0):
            so, sl = cache.slot(int(p))
            ro, rl = ref_cache.slots[p]
            assert_state_close(sel(to_host(so)), sel(to_host(sl)), ro, rl, wl.dtype,
                               f"{wl.name} step {s} fresh slot {p}")
            assert cache.info(int(p)) == (True, s)
        worst = [max(worst[0], eo), max(worst[1], el)]
        say(f"[{wl.name}] step {s}: fresh {nf}/{wl.P}  O err {eo:.2e}  LSE err {el:.2e}")
        if compose_ahead and s + 1 < steps:
            nxt = dita.dita_plan_mask(plan, s + 1, cache)
            assert np.array_equal(nxt, oracle_mask(ref_plan, s + 1, ref_cache.valid))
            assert cache.compose_runs(nxt) == oracle_compose_runs(ref_cache, nxt)
            for p in ref_cache.leaders():
                first, last = ref_cache.group_range(p)
                assert cache.group(p) == (first, last)
                if last > first:
                    so, sl = cache.slot(p)
                    ro, rl = ref_cache.slots[p]
                    assert_state_close(sel(to_host(so)), sel(to_host(sl)), ro, rl, wl.dtype,
                                       f"{wl.name} step {s} group [{first}, {last}]")
    return worst, fresh_total, (cache, q_dev, inp)


@pytest.mark.parametrize("name", ["tiny_f32", "dit16k_bf16", "dit32k_bf16"])
def test_single_step_workload(dev, name):
    wl = workloads.get(name)
    worst, fresh, _ = run_schedule(wl, dev)
    expect_fresh = {"tiny_f32": 4 + 2, "dit32k_bf16": 8 + 2}
    if name in expect_fresh:
        assert fresh == expect_fresh[name]


@pytest.mark.parametrize("compose_ahead", [False, True])
def test_dit75k_anchor_schedule(dev, compose_ahead):
    wl = workloads.get("dit75k_bf16")
    worst, fresh, _ = run_schedule(wl, dev, compose_ahead=compose_ahead)
    assert fresh == 56


def test_dit75k_ramp50_schedule(dev):
    wl = workloads.get("dit75k_ramp50")
    worst, fresh, _ = run_schedule(wl, dev, compose_ahead=True)
    assert fresh == 282


@pytest.mark.parametrize("name", ["tiny_f32", "dit16k_bf16"])
def test_step_invariants(dev, name):
    """All-reuse reproduces the previous output bitwise; all-fresh equals full attention;
    the step is deterministic."""
    import partial_state_reuse_amd as dita
    wl = workloads.get(name)
    inp = Inputs(wl, seed=5)
    _, _, (cache, q_dev, _) = run_schedule(wl, dev, steps=1, seed=5)
    k, v = inp.kv(0)
    ks, vs = partition_tensors(k, wl, dev), partition_tensors(v, wl, dev)
    fresh = np.zeros(wl.P, np.uint8)
    o1, l1, _ = dita.dita_attn_step(cache, q_dev, ks, vs, fresh, 1)
    o_full, l_full = full_attention(inp.q, split_parts(k, wl), split_parts(v, wl))
    assert_state_close(to_host(o1), to_host(l1), o_full, l_full, wl.dtype, "all-fresh vs full")
    o2, l2, _ = dita.dita_attn_step(cache, q_dev, ks, vs, fresh, 2)
    assert bool((o1 == o2).all()) and bool((l1 == l2).all()), "step not deterministic"
    k2, v2 = k + 1.0, v - 1.0
    ks2, vs2 = partition_tensors(k2, wl, dev), partition_tensors(v2, wl, dev)
    reuse = np.ones(wl.P, np.uint8)
    o3, l3, info = dita.dita_attn_step(cache, q_dev, ks2, vs2, reuse, 3)
    assert info.n_fresh == 0
    assert bool((o3 == o2).all()) and bool((l3 == l2).all()), "all-reuse changed the output"
    for p in range(wl.P):
        assert cache.info(p) == (True, 2)
