"""GPU parity of the planner statistics and of an error-planned schedule.

The contribution weights and the local state change (the DiTango page,
Methodology > 1. Anchor-Guided Selection Planner: Error Modeling and Online
Prediction) are computed by the library's kernels and compared with the fp64
oracle on the same inputs.  Then a whole schedule is planned by the library's
error-guided planner, fed by those kernels, beside the oracle's planner fed
the same measured values: the masks must agree bit for bit, the step outputs
and fresh states within the acceptance tolerances.
"""

import math

import numpy as np
import pytest

import workloads
from gpu_util import assert_state_close, say, to_dev, to_host
from oracle import StateCache as OracleCache
from oracle import attn_step as oracle_step
from oracle.error_planner import ErrorPlanner as OracleErrorPlanner
from oracle.error_planner import contributions, state_change
from workloads import Inputs, round_bf16, split_parts

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows_shape", [(1, 3, 257), (2, 5, 1000)])
def test_contrib_matches_oracle(dev, rows_shape):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(20)
    P = 7
    lses = [rng.normal(3.0, 2.0, rows_shape).astype(np.float32) for _ in range(P)]
    lses[2][0, 0, :5] = -np.inf                       # an empty partition on a few rows
    m = np.max(np.stack(lses), axis=0)
    lse = (m + np.log(np.sum(np.exp(np.stack(lses) - m), axis=0))).astype(np.float32)
    lse[0, 1, 3] = -np.inf                            # a row with no weight at all
    for p in range(P):
        lses[p][0, 1, 3] = -np.inf
    dl = [torch.from_numpy(x).to(dev) for x in lses]
    w = dita.dita_state_contrib(dl, torch.from_numpy(lse).to(dev))
    ref = contributions(lses, lse)
    got = to_host(w)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-300)) < 1e-12, (got, ref)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_state_change_matches_oracle_and_rolls(dev, dtype, D):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(21)
    shape = (1, 3, 333, D)
    a = rng.standard_normal(shape)
    b = a + 0.03 * rng.standard_normal(shape)
    if dtype == "bf16":
        a, b = round_bf16(a), round_bf16(b)
    else:
        a, b = a.astype(np.float32), b.astype(np.float32)
    a, b = a.astype(np.float64), b.astype(np.float64)     # exact widening of what the GPU holds
    da, db = to_dev(a, dtype, dev), to_dev(b, dtype, dev)
    la = torch.from_numpy(rng.standard_normal(shape[:3]).astype(np.float32)).to(dev)
    lb = torch.zeros_like(la)
    out = dita.dita_state_change(da, db)
    got = to_host(out)
    ref_num = float(np.sum((a - b) ** 2))
    ref_den = float(np.sum(b ** 2))
    assert abs(got[0] - ref_num) <= 1e-12 * ref_num and abs(got[1] - ref_den) <= 1e-12 * ref_den
    assert abs(got[2] - state_change(a, b)) <= 1e-12 * state_change(a, b)
    # roll: the new state replaces the previous one, bit for bit
    dita.dita_state_change(da, db, la, lb, roll=True, out=out)
    assert bool((db == da).all()) and bool((lb == la).all())
    assert to_host(out)[2] == pytest.approx(state_change(a, b), rel=1e-12)
    # identical states: no change; zero previous state: infinite change
    out = dita.dita_state_change(da, db)
    assert to_host(out)[2] == 0.0
    z = torch.zeros_like(db)
    assert math.isinf(to_host(dita.dita_state_change(da, z))[2])


def test_error_planned_schedule_matches_oracle(dev):
    import torch
    import partial_state_reuse_amd as dita
    wl = workloads.reduced("dit75k_ramp50", H=4, grid=(21, 15, 16), steps=20)
    P, q = wl.P, wl.q_part
    inp = Inputs(wl, seed=3)
    tdt = torch.bfloat16
    q_dev = to_dev(inp.q, "bf16", dev)
    cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, P, device=dev)
    ref = OracleCache(P)
    group, budget, anchor = 2, 0.004, 10
    planner = dita.ErrorPlanner(P, q, group, budget, anchor)
    ref_pl = OracleErrorPlanner(P, q, group, budget, anchor)
    prev_o = torch.zeros((wl.B, wl.H, wl.Nq, wl.D), dtype=tdt, device=dev)
    prev_l = torch.zeros((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
    reused_total = 0
    for s in range(wl.steps):
        k, v = inp.kv(s)
        mask, err = planner.mask(s, cache=cache)
        ref_mask, ref_err = ref_pl.mask(s, ref.valid, ref.stamp)
        assert np.array_equal(mask, ref_mask), (s, mask, ref_mask)
        assert np.array_equal(err, ref_err), s
        ks = [to_dev(np.ascontiguousarray(x), "bf16", dev) for x in split_parts(k, wl)]
        vs = [to_dev(np.ascontiguousarray(x), "bf16", dev) for x in split_parts(v, wl)]
        o, lse, info = dita.dita_attn_step(cache, q_dev, ks, vs, mask, s)
        o_ref, lse_ref, nf = oracle_step(ref, inp.q, split_parts(k, wl), split_parts(v, wl), mask, s)
        assert info.n_fresh == nf
        reused_total += P - nf
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", f"step {s} output")
        if nf == P:
            # anchor: refresh the importance weights from the fresh states
            w = cache.contrib(lse)
            w_host = to_host(w)
            slot_lses = [to_host(cache.slot(p)[1]) for p in range(P)]
            w_chk = contributions(slot_lses, to_host(lse))
            assert np.max(np.abs(w_host - w_chk)) < 1e-12
            w_ora = contributions([ref.slots[p][1] for p in range(P)], lse_ref)
            assert np.max(np.abs(w_host - w_ora)) < 1e-4     # the fp64 oracle's own weights
            assert abs(w_host.sum() - 1.0) < 1e-5
            planner.set_weights(list(w_host))
            ref_pl.set_weights(list(w_host))
        so, sl = cache.slot(q)
        new_host, prev_host = to_host(so).copy(), to_host(prev_o).copy()
        out = dita.dita_state_change(so, prev_o, sl, prev_l, roll=True)
        if s > 0:
            d = float(to_host(out)[2])
            assert d == pytest.approx(state_change(new_host, prev_host), rel=1e-12)
            planner.observe(s, d)
            ref_pl.observe(s, d)
        say(f"[error planner] step {s}: fresh {nf}/{P}  mask {''.join(map(str, mask))}")
    assert reused_total > 0


def test_state_change_is_bitwise_reproducible(dev):
    """The change statistic sums in an order fixed by the state's size alone: the
    same inputs give the same three doubles bit for bit, at the 75,600-token
    state's size (many workgroups, capped grid)."""
    import torch
    import partial_state_reuse_amd as dita
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    shape = (1, 40, 4725, 128)
    a = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    b = (a.float() + 0.03 * torch.randn(shape, generator=g, device=dev)).to(torch.bfloat16)
    outs = [dita.dita_state_change(a, b).clone() for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert bool((o == outs[0]).all()), (outs[0], o)
    ref = float(((a.double() - b.double()) ** 2).sum() / (b.double() ** 2).sum()) ** 0.5
    assert to_host(outs[0])[2] == pytest.approx(ref, rel=1e-12)


def test_error_planned_schedule_is_reproducible(dev):
    """Two runs of an error-planned schedule, the planner fed by the library's own
    statistics kernels: identical measured changes and identical masks."""
    import torch
    import partial_state_reuse_amd as dita
    wl = workloads.reduced("dit75k_ramp50", H=4, grid=(21, 15, 16), steps=12)
    P, q = wl.P, wl.q_part
    inp = Inputs(wl, seed=4)
    tdt = torch.bfloat16
    q_dev = to_dev(inp.q, "bf16", dev)
    kv = []
    for s in range(wl.steps):
        k, v = inp.kv(s)
        kv.append(([to_dev(np.ascontiguousarray(x), "bf16", dev) for x in split_parts(k, wl)],
                   [to_dev(np.ascontiguousarray(x), "bf16", dev) for x in split_parts(v, wl)]))
    runs = []
    for run in range(2):
        cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, P, device=dev)
        planner = dita.ErrorPlanner(P, q, 2, 0.004, 6)
        prev_o = torch.zeros((wl.B, wl.H, wl.Nq, wl.D), dtype=tdt, device=dev)
        prev_l = torch.zeros((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
        masks, deltas = [], []
        for s in range(wl.steps):
            mask, _ = planner.mask(s, cache=cache)
            _, lse, info = dita.dita_attn_step(cache, q_dev, kv[s][0], kv[s][1], mask, s)
            if info.n_fresh == P:
                planner.set_weights(list(to_host(cache.contrib(lse))))
            so, sl = cache.slot(q)
            out = dita.dita_state_change(so, prev_o, sl, prev_l, roll=True)
            if s > 0:
                d = float(to_host(out)[2])
                planner.observe(s, d)
                deltas.append(d)
            masks.append(mask.copy())
        runs.append((masks, deltas))
        say(f"[reproducible planner] run {run}: deltas {deltas[:3]} ...")
    assert all(np.array_equal(x, y) for x, y in zip(runs[0][0], runs[1][0]))
    assert runs[0][1] == runs[1][1]
