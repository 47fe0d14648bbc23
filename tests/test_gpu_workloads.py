"""GPU parity of whole rank-step schedules on the five synthetic workloads.

For every step: the library's mask must equal the oracle planner's bit for
bit; the fresh states written into the cache, and the merged output and LSE,
must match the oracle's within the acceptance tolerances.  The tiny, 16k and
32,760-token workloads are compared in full (every head, every query row, every
fresh state).  The 75,600-token schedules run at full size on the GPU and are
compared on every head at query rows that reach every 32-row query block
(each wave's block of the attention kernel) and the first and last row of
every 512-row tile; attention rows are independent, so the oracle restricted
to those rows is the full oracle there.  The oracle runs head by head in
threads (heads never interact).
"""

import numpy as np
import pytest

import workloads
from gpu_util import HeadChunkedOracle, assert_state_close, covering_rows, say, to_dev, to_host
from oracle import Plan as OraclePlan
from oracle import full_attention
from oracle import plan_mask as oracle_mask
from workloads import Inputs, split_parts

pytestmark = pytest.mark.gpu


def partition_tensors(x: np.ndarray, wl, dev):
    """[B, H, N, D] host array -> P contiguous [B, H, Nk, D] device tensors."""
    return [to_dev(np.ascontiguousarray(x[:, :, a:b]), wl.dtype, dev)
            for a, b in (wl.part_range(p) for p in range(wl.P))]


def sample_rows(wl):
    """Query rows compared with the oracle: all of them up to the 32,760-token
    workload, else rows reaching every query block and tile (all heads always)."""
    if wl.Nq * wl.H <= 40 * 4095:
        return None
    return covering_rows(wl.Nq)


def run_schedule(wl, dev, steps=None, seed=0, compose_ahead=False):
    """Run the workload's schedule on both sides.  With ``compose_ahead`` the
    runs of partitions the next step reuses are composed into groups after
    every step, on both sides: by ``compose_runs`` after the step, or with
    ``compose_ahead="step"`` by the step itself (``compose_next``, the
    benchmark's pipeline; the oracle composes after its step)."""
    import torch
    import partial_state_reuse_amd as dita
    steps = wl.steps if steps is None else steps
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    say(f"[{wl.name}] generating inputs H={wl.H} N={wl.N} P={wl.P}")
    inp = Inputs(wl, seed=seed)
    rows = sample_rows(wl)
    sel = (lambda x: x) if rows is None else (lambda x: x[:, :, rows])
    rows_t = None if rows is None else torch.from_numpy(rows).to(dev)

    def host(t):
        """A device tensor's compared rows, widened to float64 on the host."""
        return to_host(t if rows_t is None else t.index_select(2, rows_t))
    say(f"[{wl.name}] comparing all {wl.H} heads, "
        f"{'all' if rows is None else len(rows)} of {wl.Nq} query rows")
    q_dev = to_dev(inp.q, wl.dtype, dev)
    q_ref = sel(inp.q)
    cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev)
    ref_cache = HeadChunkedOracle(wl.P, wl.H)
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
        # every partition holds a valid state after a step: no cache for the next mask
        nxt = (dita.dita_plan_mask(plan, s + 1) if compose_ahead == "step" and s + 1 < steps
               else None)
        o, lse, info = dita.dita_attn_step(cache, q_dev, ks, vs, mask, s, compose_next=nxt)
        kp, vp = split_parts(k, wl), split_parts(v, wl)
        o_ref, lse_ref, nf = ref_cache.step(q_ref, kp, vp, mask, s)
        assert info.n_fresh == nf == int((mask == 0).sum())
        fresh_total += nf
        eo, el = assert_state_close(host(o), host(lse), o_ref, lse_ref, wl.dtype,
                                    f"{wl.name} step {s} output")
        for p in np.flatnonzero(mask == 0):
            first, last = cache.group(int(p))
            if last > first:  # composed by the step already: compared below as a group
                continue
            so, sl = cache.slot(int(p))
            ro, rl = ref_cache.slot(int(p))
            assert_state_close(host(so), host(sl), ro, rl, wl.dtype,
                               f"{wl.name} step {s} fresh slot {p}")
            assert cache.info(int(p)) == (True, s)
        worst = [max(worst[0], eo), max(worst[1], el)]
        say(f"[{wl.name}] step {s}: fresh {nf}/{wl.P}  O err {eo:.2e}  LSE err {el:.2e}")
        if compose_ahead and s + 1 < steps:
            if nxt is None:
                nxt = dita.dita_plan_mask(plan, s + 1, cache)
                assert np.array_equal(nxt, oracle_mask(ref_plan, s + 1, ref_cache.valid))
                assert cache.compose_runs(nxt) == ref_cache.compose_runs(nxt)
            else:
                assert np.array_equal(nxt, oracle_mask(ref_plan, s + 1, ref_cache.valid))
                assert info.composed == ref_cache.compose_runs(nxt)
            for p in ref_cache.leaders():
                first, last = ref_cache.group_range(p)
                assert cache.group(p) == (first, last)
                if last > first:
                    so, sl = cache.slot(p)
                    ro, rl = ref_cache.slot(p)
                    assert_state_close(host(so), host(sl), ro, rl, wl.dtype,
                                       f"{wl.name} step {s} group [{first}, {last}]")
    return worst, fresh_total, (cache, q_dev, inp)


@pytest.mark.parametrize("name", ["tiny_f32", "dit16k_bf16", "dit32k_bf16"])
def test_single_step_workload(dev, name):
    wl = workloads.get(name)
    worst, fresh, _ = run_schedule(wl, dev)
    expect_fresh = {"tiny_f32": 4 + 2, "dit32k_bf16": 8 + 2}
    if name in expect_fresh:
        assert fresh == expect_fresh[name]


@pytest.mark.parametrize("compose_ahead", [False, True, "step"])
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


def test_dit75k_lone_block_partial(dev):
    """One dita_attn_partial call on one 75,600-token block (the rank's 4725
    queries against partition 5's 4725 keys, all 40 heads), the launch the
    planner lays out staged on a 256-CU device (255 512-row tiles, then 250
    256-row tiles): all heads at rows reaching every query block and tile,
    against the oracle's partial state."""
    import partial_state_reuse_amd as dita
    from oracle import partial_state
    wl = workloads.get("dit75k_bf16")
    lay = dita.dita_attn_launch_info(wl.B, wl.H, wl.Nq, wl.D, 1, wl.Nk)
    say(f"[{wl.name}] lone block layout={lay}")
    if lay["compute_units"] == 256:
        assert lay["staged_pairs"] >= 0 and lay["split_units"] == 0, lay
    inp = Inputs(wl, seed=3)
    k, v = inp.kv(0)
    a, b = wl.part_range(5)
    kp, vp = np.ascontiguousarray(k[:, :, a:b]), np.ascontiguousarray(v[:, :, a:b])
    del k, v
    o, lse = dita.dita_attn_partial(to_dev(inp.q, wl.dtype, dev), to_dev(kp, wl.dtype, dev),
                                    to_dev(vp, wl.dtype, dev))
    rows = covering_rows(wl.Nq)
    o_ref, lse_ref = partial_state(np.ascontiguousarray(inp.q[:, :, rows]), kp, vp)
    import torch
    rows_t = torch.from_numpy(rows).to(dev)
    assert_state_close(to_host(o.index_select(2, rows_t)), to_host(lse.index_select(2, rows_t)),
                       o_ref, lse_ref, wl.dtype, "lone 75,600-token block")
