"""C-ABI checks that need no GPU: exports, planner bit-parity, argument validation.

Every call made here either touches host metadata only (the planner, the
cache handle) or is rejected by validation before the library makes any HIP
call, so nothing is launched.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import workloads
from oracle import Plan as OraclePlan
from oracle import plan_mask as oracle_plan_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

dita = pytest.importorskip("partial_state_reuse_amd")
lib = dita.lib()

FAKE_DEV = 0x7F0000000000  # an aligned address that is never dereferenced here


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "dita.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dita_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert lib.dita_status_str(0) == b"ok"
    assert b"align" in lib.dita_status_str(dita.DITA_ERR_ALIGN)
    assert lib.dita_status_str(99) == b"unknown status"
    assert lib.dita_version() >= 100


def _lib_mask(plan: OraclePlan, step):
    cp = dita.Plan(plan.P, plan.q, plan.policy, plan.radius, plan.radius_end, plan.k_nearest,
                   plan.anchor_period, plan.total_steps, plan.seed)
    out = (ctypes.c_uint8 * plan.P)()
    assert lib.dita_plan_mask(ctypes.byref(cp), None, step, out) == 0
    return np.frombuffer(bytes(out), np.uint8)


def _cache(shape, P):
    h = ctypes.c_void_p()
    n = lib.dita_state_cache_bytes(ctypes.byref(shape), P)
    assert lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(shape), P, FAKE_DEV, n) == 0
    return h.value


@pytest.mark.parametrize("name", workloads.ORDER)
def test_planner_matches_oracle_on_workload_schedules(name):
    wl = workloads.get(name)
    plan = OraclePlan(**wl.plan_fields())
    for s in range(wl.steps):
        assert np.array_equal(_lib_mask(plan, s), oracle_plan_mask(plan, s)), (name, s)


def test_planner_matches_oracle_on_random_plans():
    rng = np.random.default_rng(1234)
    for _ in range(10000):
        P = int(rng.integers(1, 65))
        plan = OraclePlan(P=P, q=int(rng.integers(0, P)), policy=int(rng.integers(0, 4)),
                          radius=int(rng.integers(0, 70)), radius_end=int(rng.integers(0, 70)),
                          k_nearest=int(rng.integers(0, P + 2)),
                          anchor_period=int(rng.integers(0, 7)),
                          total_steps=int(rng.integers(1, 100)),
                          seed=int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)))
        s = int(rng.integers(0, 200))
        assert np.array_equal(_lib_mask(plan, s), oracle_plan_mask(plan, s)), (plan, s)


def test_planner_bitmask_encoding_matches_oracle():
    """The 64-bit mask encoding: bit p of the word is byte p of the oracle's mask."""
    rng = np.random.default_rng(5)
    for trial in range(500):
        P = int(rng.integers(1, 65))
        plan = OraclePlan(P=P, q=int(rng.integers(0, P)), policy=int(rng.integers(0, 4)),
                          radius=int(rng.integers(0, 10)), radius_end=int(rng.integers(0, 10)),
                          k_nearest=int(rng.integers(0, P + 1)), anchor_period=int(rng.integers(0, 6)),
                          total_steps=int(rng.integers(1, 60)), seed=int(rng.integers(0, 2**32)))
        step = int(rng.integers(0, 60))
        ref = oracle_plan_mask(plan, step)
        want = sum(int(b) << p for p, b in enumerate(ref))
        cp = dita.Plan(plan.P, plan.q, plan.policy, plan.radius, plan.radius_end, plan.k_nearest,
                       plan.anchor_period, plan.total_steps, plan.seed)
        assert dita.dita_plan_bits(cp, step) == want, trial
        back = (ctypes.c_uint8 * P)()
        assert lib.dita_mask_from_bits(want, P, back) == 0 and list(back) == list(ref)
        bits = ctypes.c_uint64()
        assert lib.dita_mask_to_bits((ctypes.c_uint8 * P)(*ref), P, ctypes.byref(bits)) == 0
        assert bits.value == want
    out = (ctypes.c_uint8 * 4)()
    assert lib.dita_mask_from_bits(1 << 4, 4, out) == dita.DITA_ERR_ARG      # a bit past P
    assert lib.dita_mask_to_bits((ctypes.c_uint8 * 4)(0, 2, 0, 0), 4, ctypes.byref(ctypes.c_uint64())) == dita.DITA_ERR_ARG
    assert lib.dita_mask_from_bits(0, 65, out) == dita.DITA_ERR_ARG
    full = (ctypes.c_uint8 * 64)()
    assert lib.dita_mask_from_bits(2**64 - 1, 64, full) == 0 and sum(full) == 64


def test_planner_rejects_bad_plans():
    out = (ctypes.c_uint8 * 64)()
    for bad in [dita.Plan(0, 0, 0, 0, 0, 0, 0, 1, 0), dita.Plan(65, 0, 0, 0, 0, 0, 0, 1, 0),
                dita.Plan(4, 4, 0, 0, 0, 0, 0, 1, 0), dita.Plan(4, 0, 9, 0, 0, 0, 0, 1, 0),
                dita.Plan(4, 0, 0, -1, 0, 0, 0, 1, 0), dita.Plan(4, 0, 3, 0, 0, 0, 0, 0, 0),
                dita.Plan(4, 0, 0, 0, 0, -2, 0, 1, 0), dita.Plan(4, 0, 0, 0, 0, 0, -1, 1, 0)]:
        assert lib.dita_plan_mask(ctypes.byref(bad), None, 0, out) == dita.DITA_ERR_ARG
    ok = dita.Plan(4, 0, 0, 0, 0, 0, 0, 1, 0)
    assert lib.dita_plan_mask(ctypes.byref(ok), None, -1, out) == dita.DITA_ERR_ARG
    assert lib.dita_plan_mask(ctypes.byref(ok), None, 0, None) == dita.DITA_ERR_ARG


def test_cache_metadata_host_only():
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 100, 0.0)
    n = lib.dita_state_cache_bytes(ctypes.byref(shape), 3)
    o_bytes = 1 * 2 * 100 * 128 * 2
    lse_bytes = 1 * 2 * 100 * 4
    align = lambda x: (x + 255) // 256 * 256
    assert n == 3 * (align(o_bytes) + align(lse_bytes))
    h = _cache(shape, 3)
    o, l = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.dita_state_cache_slot(h, 2, ctypes.byref(o), ctypes.byref(l)) == 0
    assert o.value == FAKE_DEV + 2 * (align(o_bytes) + align(lse_bytes))
    assert l.value == o.value + align(o_bytes)
    valid, stamp = ctypes.c_int(), ctypes.c_int64()
    for p in range(3):
        assert lib.dita_state_cache_info(h, p, ctypes.byref(valid), ctypes.byref(stamp)) == 0
        assert valid.value == 0 and stamp.value == -1
    assert lib.dita_state_cache_info(h, 3, None, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_invalidate(h, -1) == 0
    assert lib.dita_state_cache_invalidate(h, 5) == dita.DITA_ERR_ARG
    sh, P = dita.Shape(), ctypes.c_int()
    assert lib.dita_state_cache_shape(h, ctypes.byref(sh), ctypes.byref(P)) == 0
    assert (sh.B, sh.H, sh.D, sh.Nq, P.value) == (1, 2, 128, 100, 3)
    # Loading an empty slot is a state error, detected before any copy is issued.
    assert lib.dita_state_cache_load(h, 0, FAKE_DEV, FAKE_DEV + 4096, None) == dita.DITA_ERR_STATE
    # The planner honours cold slots: with every slot empty, everything is fresh.
    plan = dita.Plan(3, 0, dita.DITA_PLAN_DIST, 0, 0, 0, 0, 1, 0)
    out = (ctypes.c_uint8 * 3)()
    assert lib.dita_plan_mask(ctypes.byref(plan), h, 4, out) == 0
    assert list(out) == [0, 0, 0]
    plan4 = dita.Plan(4, 0, dita.DITA_PLAN_DIST, 0, 0, 0, 0, 1, 0)
    assert lib.dita_plan_mask(ctypes.byref(plan4), h, 4, out) == dita.DITA_ERR_ARG  # P mismatch
    lib.dita_state_cache_free(h)
    assert lib.dita_state_cache_free(None) == 0


def test_cache_init_validation():
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 100, 0.0)
    n = lib.dita_state_cache_bytes(ctypes.byref(shape), 3)
    h = ctypes.c_void_p()
    assert lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(shape), 3, FAKE_DEV, n - 1) == dita.DITA_ERR_SIZE
    assert lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(shape), 0, FAKE_DEV, n) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(shape), 65, FAKE_DEV, n) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(shape), 3, FAKE_DEV + 8, n) == dita.DITA_ERR_ALIGN
    assert lib.dita_state_cache_init(ctypes.byref(h), ctypes.byref(shape), 3, None, n) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_init(None, ctypes.byref(shape), 3, FAKE_DEV, n) == dita.DITA_ERR_ARG
    assert h.value is None
    assert lib.dita_state_cache_bytes(None, 3) == 0
    bad = dita.Shape(1, 2, 96, dita.DITA_BF16, 100, 0.0)
    assert lib.dita_state_cache_bytes(ctypes.byref(bad), 3) == 0


@pytest.mark.parametrize("field,value,status", [
    ("D", 96, dita.DITA_ERR_SHAPE), ("D", 256, dita.DITA_ERR_SHAPE), ("B", 0, dita.DITA_ERR_SHAPE),
    ("H", 70000, dita.DITA_ERR_SHAPE), ("Nq", 0, dita.DITA_ERR_SHAPE),
    ("Nq", 2**31, dita.DITA_ERR_SHAPE), ("dtype", 5, dita.DITA_ERR_DTYPE),
    ("scale", float("nan"), dita.DITA_ERR_ARG), ("scale", float("inf"), dita.DITA_ERR_ARG),
])
def test_attn_partial_rejects_bad_shape(field, value, status):
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 64, 0.0)
    setattr(shape, field, value)
    p = FAKE_DEV
    assert lib.dita_attn_partial(ctypes.byref(shape), p, p, p, 64, p, p, None) == status


def test_attn_partial_rejects_bad_pointers_and_nk():
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 64, 0.0)
    p = FAKE_DEV
    assert lib.dita_attn_partial(None, p, p, p, 64, p, p, None) == dita.DITA_ERR_ARG
    assert lib.dita_attn_partial(ctypes.byref(shape), None, p, p, 64, p, p, None) == dita.DITA_ERR_ARG
    assert lib.dita_attn_partial(ctypes.byref(shape), p, p + 2, p, 64, p, p, None) == dita.DITA_ERR_ALIGN
    assert lib.dita_attn_partial(ctypes.byref(shape), p, p, p, 64, p, p + 4, None) == dita.DITA_ERR_ALIGN
    assert lib.dita_attn_partial(ctypes.byref(shape), p, p, p, 0, p, p, None) == dita.DITA_ERR_SHAPE
    assert lib.dita_attn_partial(ctypes.byref(shape), p, p, p, 2**31, p, p, None) == dita.DITA_ERR_SHAPE
    # one head's K slice must stay below 2^31 bytes: 2^23 keys x 128 x 2 bytes is 2^31
    assert lib.dita_attn_partial(ctypes.byref(shape), p, p, p, 2**23, p, p, None) == dita.DITA_ERR_SHAPE
    f32 = dita.Shape(1, 2, 128, dita.DITA_F32, 64, 0.0)
    assert lib.dita_attn_partial(ctypes.byref(f32), p, p, p, 2**22, p, p, None) == dita.DITA_ERR_SHAPE


def test_state_merge_rejects_bad_arguments():
    shape = dita.Shape(1, 2, 64, dita.DITA_F32, 64, 0.0)
    p = FAKE_DEV
    arr = lambda *x: (ctypes.c_void_p * len(x))(*x)
    o_bytes = 2 * 64 * 64 * 4
    srcs = arr(p, p + (1 << 20))
    lses = arr(p + (2 << 20), p + (3 << 20))
    out, out_l = p + (4 << 20), p + (5 << 20)
    assert lib.dita_state_merge(ctypes.byref(shape), 0, srcs, lses, out, out_l, None) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_merge(ctypes.byref(shape), 65, srcs, lses, out, out_l, None) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_merge(ctypes.byref(shape), 2, None, lses, out, out_l, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_merge(ctypes.byref(shape), 2, arr(p, p + 8), lses, out, out_l, None) == dita.DITA_ERR_ALIGN
    assert lib.dita_state_merge(ctypes.byref(shape), 2, arr(p, None), lses, out, out_l, None) == dita.DITA_ERR_ARG
    # output aliasing an input state
    assert lib.dita_state_merge(ctypes.byref(shape), 2, arr(p, p + (1 << 20)), lses, p + 256, out_l,
                                None) == dita.DITA_ERR_ARG
    assert o_bytes < (1 << 20)


def test_attn_step_validation_before_launch():
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 64, 0.0)
    h = _cache(shape, 4)
    n = lib.dita_state_cache_bytes(ctypes.byref(shape), 4)
    q, o, l = FAKE_DEV + n + 4096, FAKE_DEV + n + (1 << 20), FAKE_DEV + n + (2 << 20)
    ks = (ctypes.c_void_p * 4)(*[FAKE_DEV + n + ((3 + i) << 20) for i in range(4)])
    nk = (ctypes.c_int64 * 4)(64, 64, 64, 64)
    mask = lambda *m: (ctypes.c_uint8 * 4)(*m)
    info = dita.StepInfo()
    # Reusing a slot that was never filled.
    assert lib.dita_attn_step(h, q, ks, ks, nk, mask(0, 1, 0, 0), 0, o, l, None, ctypes.byref(info)) == dita.DITA_ERR_STATE
    # Mask values other than 0/1.
    assert lib.dita_attn_step(h, q, ks, ks, nk, mask(0, 2, 0, 0), 0, o, l, None, None) == dita.DITA_ERR_ARG
    # Output inside the cache buffer.
    assert lib.dita_attn_step(h, q, ks, ks, nk, mask(0, 0, 0, 0), 0, FAKE_DEV + 256, l, None, None) == dita.DITA_ERR_ARG
    # Bad key count of a fresh partition.
    bad_nk = (ctypes.c_int64 * 4)(64, 0, 64, 64)
    assert lib.dita_attn_step(h, q, ks, ks, bad_nk, mask(0, 0, 0, 0), 0, o, l, None, None) == dita.DITA_ERR_SHAPE
    # Misaligned K of a fresh partition.
    bad_k = (ctypes.c_void_p * 4)(ks[0], ks[1] + 2, ks[2], ks[3])
    assert lib.dita_attn_step(h, q, bad_k, ks, nk, mask(0, 0, 0, 0), 0, o, l, None, None) == dita.DITA_ERR_ALIGN
    # Negative step, null handle, null lists.
    assert lib.dita_attn_step(h, q, ks, ks, nk, mask(0, 0, 0, 0), -1, o, l, None, None) == dita.DITA_ERR_ARG
    assert lib.dita_attn_step(None, q, ks, ks, nk, mask(0, 0, 0, 0), 0, o, l, None, None) == dita.DITA_ERR_ARG
    assert lib.dita_attn_step(h, q, None, ks, nk, mask(0, 0, 0, 0), 0, o, l, None, None) == dita.DITA_ERR_ARG
    # Nothing changed.
    valid, stamp = ctypes.c_int(), ctypes.c_int64()
    for p in range(4):
        lib.dita_state_cache_info(h, p, ctypes.byref(valid), ctypes.byref(stamp))
        assert valid.value == 0 and stamp.value == -1
    lib.dita_state_cache_free(h)


def test_group_calls_host_only():
    """Group metadata calls on an empty cache: every partition is a group of one,
    and composition of states that do not exist is refused before any launch."""
    shape = dita.Shape(1, 2, 64, dita.DITA_BF16, 64, 0.0)
    h = _cache(shape, 5)
    a, b = ctypes.c_int(), ctypes.c_int()
    for p in range(5):
        assert lib.dita_state_cache_group(h, p, ctypes.byref(a), ctypes.byref(b)) == 0
        assert (a.value, b.value) == (p, p)
    assert lib.dita_state_cache_group(h, 5, None, None) == dita.DITA_ERR_ARG
    live = ctypes.c_int()
    assert lib.dita_state_cache_live(h, ctypes.byref(live)) == 0 and live.value == 0
    assert lib.dita_state_cache_live(h, None) == dita.DITA_ERR_ARG
    for first, last in [(2, 1), (-1, 2), (0, 5)]:
        assert lib.dita_state_cache_compose(h, first, last, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_compose(h, 1, 3, None) == dita.DITA_ERR_STATE
    assert lib.dita_state_cache_compose(None, 0, 1, None) == dita.DITA_ERR_ARG
    m = (ctypes.c_uint8 * 5)(0, 0, 0, 0, 0)
    out = (ctypes.c_uint8 * 5)(9, 9, 9, 9, 9)
    assert lib.dita_state_cache_effective_mask(h, m, out) == 0 and list(out) == [0] * 5
    assert lib.dita_state_cache_effective_mask(h, (ctypes.c_uint8 * 5)(0, 1, 0, 0, 0), out) == dita.DITA_ERR_STATE
    assert lib.dita_state_cache_effective_mask(h, (ctypes.c_uint8 * 5)(0, 3, 0, 0, 0), out) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_effective_mask(h, None, out) == dita.DITA_ERR_ARG
    lib.dita_state_cache_free(h)


def test_attn_step_ex_validates_options():
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 64, 0.0)
    h = _cache(shape, 2)
    n = lib.dita_state_cache_bytes(ctypes.byref(shape), 2)
    q, o, l = FAKE_DEV + n + 4096, FAKE_DEV + n + (1 << 20), FAKE_DEV + n + (2 << 20)
    ks = (ctypes.c_void_p * 2)(FAKE_DEV + n + (3 << 20), FAKE_DEV + n + (4 << 20))
    nk = (ctypes.c_int64 * 2)(64, 64)
    zeros = (ctypes.c_uint8 * 2)(0, 0)
    for side, minp, res in [(FAKE_DEV, 0, 1), (FAKE_DEV, -1, 0)]:
        opts = dita.StepOpts(side, minp, res)
        assert lib.dita_attn_step_ex(h, q, ks, ks, nk, zeros, 0, o, l, None, ctypes.byref(opts),
                                     None) == dita.DITA_ERR_ARG
    opts = dita.StepOpts(FAKE_DEV, 0, 0)
    assert lib.dita_attn_step_ex(h, q, ks, ks, nk, (ctypes.c_uint8 * 2)(0, 1), 0, o, l, None,
                                 ctypes.byref(opts), None) == dita.DITA_ERR_STATE
    # compose_next holds 0/1 values only: rejected before anything is enqueued
    bad = (ctypes.c_uint8 * 2)(0, 2)
    opts = dita.StepOpts(None, 0, 0, ctypes.cast(bad, ctypes.POINTER(ctypes.c_uint8)))
    assert lib.dita_attn_step_ex(h, q, ks, ks, nk, zeros, 0, o, l, None, ctypes.byref(opts),
                                 None) == dita.DITA_ERR_ARG
    lib.dita_state_cache_free(h)


def test_error_planner_matches_oracle_bit_for_bit():
    """The C++ error-guided planner against the oracle's, on random weights,
    observations (in any order, some replaced), stamps, validity, group sizes and
    budgets: the masks must agree exactly and the error estimates to the bit."""
    from oracle.error_planner import ErrorPlanner as OracleErrorPlanner
    rng = np.random.default_rng(42)
    n_reused = 0
    for trial in range(3000):
        P = int(rng.integers(1, 65))
        q = int(rng.integers(0, P))
        g = int(rng.integers(1, 6))
        ap = int(rng.choice([0, 0, 3, 5, 7]))
        budget = float(rng.choice([0.0, rng.uniform(0, 0.02), rng.uniform(0, 0.2), np.inf]))
        fw = float(rng.choice([0.0, 0.0, rng.uniform(0.02, 0.2)]))
        ref = OracleErrorPlanner(P, q, g, budget, ap, fw)
        lib_pl = dita.ErrorPlanner(P, q, g, budget, ap, fw)
        if rng.random() < 0.95:
            w = rng.dirichlet(np.ones(P) * 0.5)
            ref.set_weights(list(w))
            lib_pl.set_weights(list(w))
        step = int(rng.integers(0, 40))
        for _ in range(int(rng.integers(0, 8))):
            t = int(rng.integers(0, 45))
            d = float(rng.choice([0.0, rng.exponential(0.01)]))
            ref.observe(t, d)
            lib_pl.observe(t, d)
        valid = (rng.random(P) < 0.9).astype(np.uint8)
        stamp = np.where(valid == 1, rng.integers(0, step + 1, P), -1)
        r_ref, e_ref = ref.mask(step, valid, stamp)
        r_lib, e_lib = lib_pl.mask(step, valid, stamp)
        assert np.array_equal(r_ref, r_lib), (trial, r_ref, r_lib)
        assert np.array_equal(e_ref, e_lib), (trial, e_ref, e_lib)
        n_reused += int(r_ref.sum())
    assert n_reused > 1000          # the random plans do reuse


def test_error_planner_validation():
    bad = [(0, 0, 1, 0, 0.1, 0.0), (4, 4, 1, 0, 0.1, 0.0), (4, 0, 0, 0, 0.1, 0.0),
           (4, 0, 1, -1, 0.1, 0.0), (4, 0, 1, 0, -0.5, 0.0), (4, 0, 1, 0, float("nan"), 0.0),
           (4, 0, 1, 0, 0.1, -0.2), (4, 0, 1, 0, 0.1, float("nan"))]
    h = ctypes.c_void_p()
    for args in bad:
        assert lib.dita_planner_create(ctypes.byref(h), ctypes.byref(dita.ErrorPlan(*args))) == dita.DITA_ERR_ARG
    assert lib.dita_planner_create(None, ctypes.byref(dita.ErrorPlan(4, 0, 1, 0, 0.1, 0.0))) == dita.DITA_ERR_ARG
    pl = dita.ErrorPlanner(4, 0, 2, 0.1)
    dbl = lambda *x: (ctypes.c_double * 4)(*x)
    assert lib.dita_planner_set_weights(pl.handle, dbl(0.1, -0.1, 0.5, 0.5)) == dita.DITA_ERR_ARG
    assert lib.dita_planner_set_weights(pl.handle, dbl(0.1, float("inf"), 0.5, 0.5)) == dita.DITA_ERR_ARG
    assert lib.dita_planner_observe(pl.handle, -1, 0.1) == dita.DITA_ERR_ARG
    assert lib.dita_planner_observe(pl.handle, 2, float("nan")) == dita.DITA_ERR_ARG
    assert lib.dita_planner_observe(pl.handle, 2, -1.0) == dita.DITA_ERR_ARG
    v = (ctypes.c_uint8 * 4)(1, 1, 1, 1)
    out = (ctypes.c_uint8 * 4)()
    t_bad = (ctypes.c_int64 * 4)(0, 0, 9, 0)        # a stamp after the planned step
    assert lib.dita_planner_mask(pl.handle, 5, v, t_bad, out, None) == dita.DITA_ERR_ARG
    v_bad = (ctypes.c_uint8 * 4)(1, 2, 1, 1)
    t_ok = (ctypes.c_int64 * 4)(0, 0, 0, 0)
    assert lib.dita_planner_mask(pl.handle, 5, v_bad, t_ok, out, None) == dita.DITA_ERR_ARG
    assert lib.dita_planner_mask(pl.handle, 5, v, t_ok, out, None) == 0
    assert lib.dita_planner_free(None) == 0


def test_stats_calls_validate_before_launch():
    shape = dita.Shape(1, 2, 64, dita.DITA_BF16, 64, 0.0)
    p = FAKE_DEV
    arr = lambda *x: (ctypes.c_void_p * len(x))(*x)
    l2 = arr(p, p + 4096)
    assert lib.dita_state_contrib(ctypes.byref(shape), 0, l2, p + 8192, p + 16384, None) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_contrib(ctypes.byref(shape), 2, None, p + 8192, p + 16384, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_contrib(ctypes.byref(shape), 2, arr(p, p + 4), p + 8192, p + 16384, None) == dita.DITA_ERR_ALIGN
    assert lib.dita_state_contrib(ctypes.byref(shape), 2, l2, p + 8192, None, None) == dita.DITA_ERR_ARG
    o_bytes = 2 * 64 * 64 * 2
    a, b, out = p, p + (1 << 20), p + (2 << 20)
    assert lib.dita_state_change(ctypes.byref(shape), a, None, a + 256, None, 0, out, None) == dita.DITA_ERR_ARG  # overlap
    assert lib.dita_state_change(ctypes.byref(shape), a, None, b, None, 2, out, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_change(ctypes.byref(shape), a, None, b, None, 1, out, None) == dita.DITA_ERR_ARG  # roll needs LSEs
    assert lib.dita_state_change(ctypes.byref(shape), a, None, b, None, 0, a + 64, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_change(ctypes.byref(shape), a, None, b, None, 0, None, None) == dita.DITA_ERR_ARG
    assert o_bytes < (1 << 20)
    h = _cache(shape, 3)
    assert lib.dita_state_cache_contrib(h, p + (64 << 20), p + (65 << 20), None) == dita.DITA_ERR_STATE
    assert lib.dita_state_cache_contrib(None, p, p, None) == dita.DITA_ERR_ARG
    pl = dita.ErrorPlanner(3, 0, 1, 0.1)
    r, e = pl.mask(3, cache=type("C", (), {"handle": h})())
    assert list(r) == [0, 0, 0]
    lib.dita_state_cache_free(h)


def test_pooled_cache_host_only():
    """Pooled cache: sizes, slot lookup, and the slot shortage a step detects before
    any launch; offload/fetch refuse states that do not exist."""
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 64, 0.0)
    h = ctypes.c_void_p()
    n2 = lib.dita_state_cache_bytes(ctypes.byref(shape), 2)
    assert lib.dita_state_cache_init_pool(ctypes.byref(h), ctypes.byref(shape), 4, 5, FAKE_DEV, n2 * 4) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_cache_init_pool(ctypes.byref(h), ctypes.byref(shape), 4, 0, FAKE_DEV, n2) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_cache_init_pool(ctypes.byref(h), ctypes.byref(shape), 4, 2, FAKE_DEV, n2 - 1) == dita.DITA_ERR_SIZE
    assert lib.dita_state_cache_init_pool(ctypes.byref(h), ctypes.byref(shape), 4, 2, FAKE_DEV, n2) == 0
    hp = h.value
    o, l = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.dita_state_cache_slot(hp, 0, ctypes.byref(o), ctypes.byref(l)) == dita.DITA_ERR_STATE
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.dita_state_cache_residency(hp, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 0
    assert (a.value, b.value, c.value) == (0, 0, 2)
    # four fresh partitions need four slots; the pool has two
    base = FAKE_DEV + (64 << 20)
    q, out, lse = base, base + (1 << 20), base + (2 << 20)
    ks = (ctypes.c_void_p * 4)(*[base + ((3 + i) << 20) for i in range(4)])
    nk = (ctypes.c_int64 * 4)(64, 64, 64, 64)
    zeros = (ctypes.c_uint8 * 4)(0, 0, 0, 0)
    assert lib.dita_attn_step(hp, q, ks, ks, nk, zeros, 0, out, lse, None, None) == dita.DITA_ERR_SIZE
    host = base + (9 << 20)
    assert lib.dita_state_cache_offload(hp, 0, host, host + 4096, None) == dita.DITA_ERR_STATE
    assert lib.dita_state_cache_offload(hp, 0, None, host, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_fetch(hp, 0, None) == dita.DITA_ERR_STATE
    assert lib.dita_state_cache_fetch(hp, 4, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_residency(None, None, None, None) == dita.DITA_ERR_ARG
    lib.dita_state_cache_free(hp)


def test_event_helpers_validate():
    assert lib.dita_event_create(None) == dita.DITA_ERR_ARG
    assert lib.dita_event_record(None, None) == dita.DITA_ERR_ARG
    assert lib.dita_event_elapsed_ms(None, None, None) == dita.DITA_ERR_ARG
    assert lib.dita_event_destroy(None) == 0


def test_attn_step_ex_rejects_output_aliasing_inputs_with_side_stream():
    """With a side stream, (o, lse) may not share memory with q or a fresh K/V:
    the pre-merge would write them while the attention reads those.  Without a
    side stream the same aliasing is accepted (validation passes up to the point
    where the fake pointers would be used, so it is not launched here)."""
    shape = dita.Shape(1, 2, 128, dita.DITA_BF16, 64, 0.0)
    h = _cache(shape, 2)
    n = lib.dita_state_cache_bytes(ctypes.byref(shape), 2)
    base = FAKE_DEV + n + 4096
    q = base
    kv = [base + (1 << 20), base + (2 << 20)]
    ks = (ctypes.c_void_p * 2)(*kv)
    vs = (ctypes.c_void_p * 2)(base + (3 << 20), base + (4 << 20))
    nk = (ctypes.c_int64 * 2)(64, 64)
    fresh = (ctypes.c_uint8 * 2)(0, 0)
    side = dita.StepOpts(FAKE_DEV + 64, 0, 0)
    lse_ok = base + (6 << 20)
    for o, l in [(q, lse_ok), (kv[1] + 256, lse_ok), (base + (5 << 20), q + 64),
                 (base + (5 << 20), vs[0] + 1024)]:
        assert lib.dita_attn_step_ex(h, q, ks, vs, nk, fresh, 0, o, l, None, ctypes.byref(side),
                                     None) == dita.DITA_ERR_ARG
    for p in range(2):
        valid = ctypes.c_int()
        lib.dita_state_cache_info(h, p, ctypes.byref(valid), None)
        assert valid.value == 0
    lib.dita_state_cache_free(h)


def _no_c_calls(monkeypatch, names):
    def boom(*a, **k):
        raise AssertionError("the C library was called")
    for n in names:
        monkeypatch.setattr(dita._lib, n, boom)


def test_binding_rejects_mismatched_tensors_before_calling(monkeypatch):
    """Every wrapper checks shapes and dtypes against each other and against the
    cache before it passes a pointer: a short or mistyped buffer raises ValueError
    and nothing reaches the library."""
    import torch
    _no_c_calls(monkeypatch, ["dita_attn_partial", "dita_state_merge", "dita_attn_step",
                              "dita_attn_step_ex", "dita_state_cache_store",
                              "dita_state_cache_load", "dita_state_cache_contrib",
                              "dita_state_contrib", "dita_state_change"])
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(1, 2, 64, 128, dtype=bf)
    k = torch.zeros(1, 2, 96, 128, dtype=bf)
    bad = [
        lambda: dita.dita_attn_partial(q, k, torch.zeros(1, 2, 95, 128, dtype=bf)),
        lambda: dita.dita_attn_partial(q, k, k.float()),
        lambda: dita.dita_attn_partial(q, torch.zeros(1, 2, 96, 64, dtype=bf), k),
        lambda: dita.dita_attn_partial(q, k, k, o=torch.zeros(1, 2, 63, 128, dtype=bf)),
        lambda: dita.dita_attn_partial(q, k, k, lse=torch.zeros(1, 2, 64, dtype=bf)),
        lambda: dita.dita_state_merge([q, q], [torch.zeros(1, 2, 64), torch.zeros(1, 2, 64)],
                                      o=torch.zeros(1, 2, 64, 64, dtype=bf)),
        lambda: dita.dita_state_merge([q, q[:, :1]], [torch.zeros(1, 2, 64)] * 2),
        lambda: dita.dita_state_contrib([torch.zeros(1, 2, 64)], torch.zeros(1, 2, 64),
                                        w=torch.zeros(2, dtype=torch.float64)),
        lambda: dita.dita_state_change(q, q[:, :, :32]),
        lambda: dita.dita_state_change(q, q, out=torch.zeros(2, dtype=torch.float64)),
        lambda: dita.dita_state_change(q, q, roll=True),
    ]
    cache = dita.StateCache(1, 2, 64, 128, bf, P=2, device="cpu")
    lse = torch.zeros(1, 2, 64, dtype=f32)
    bad += [
        lambda: cache.store(0, q[:, :, :32], lse, step=0),
        lambda: cache.store(0, q.float(), lse, step=0),
        lambda: cache.store(0, q, lse[:, :1], step=0),
        lambda: cache.load(0, o=q.float()),
        lambda: cache.contrib(lse.double()),
        lambda: dita.dita_attn_step(cache, q[:, :1], [k, k], [k, k], [0, 0], 0),
        lambda: dita.dita_attn_step(cache, q, [k, k], [k, k[:, :, :50]], [0, 0], 0),
        lambda: dita.dita_attn_step(cache, q, [k, None], [k, k], [0, 0], 0),
        lambda: dita.dita_attn_step(cache, q, [k, k.float()], [k, k.float()], [0, 0], 0),
        lambda: dita.dita_attn_step(cache, q, [k, torch.zeros(1, 2, 96, 64, dtype=bf)],
                                    [k, torch.zeros(1, 2, 96, 64, dtype=bf)], [0, 0], 0),
        lambda: dita.dita_attn_step(cache, q, [k, k], [k, k], [0, 0], 0, o=q.float()),
        lambda: dita.dita_attn_step(cache, q, [k, k], [k, k], [0, 0], 0, lse=lse[:, :, :10]),
    ]
    for i, fn in enumerate(bad):
        with pytest.raises(ValueError):
            fn()
    cache.close()


def test_compact_cache_host_only():
    """Compact-cache geometry and validation: bf16 only, S + C <= 64, the buffer size,
    and compaction of a slot without a full device state refused before any launch."""
    bf = dita.Shape(1, 2, 128, dita.DITA_BF16, 100, 0.0)
    f32 = dita.Shape(1, 2, 128, dita.DITA_F32, 100, 0.0)
    rows = 2 * 100
    full = lib.dita_state_cache_bytes(ctypes.byref(bf), 3)
    a256 = lambda x: (x + 255) // 256 * 256
    per_compact = a256(rows * 128) + 2 * a256(rows * 4)
    assert lib.dita_state_cache_bytes_compact(ctypes.byref(bf), 3, 4) == full + 4 * per_compact
    assert lib.dita_state_cache_bytes_compact(ctypes.byref(bf), 3, 0) == full
    assert lib.dita_state_cache_bytes_compact(ctypes.byref(f32), 3, 1) == 0
    assert lib.dita_state_cache_bytes_compact(ctypes.byref(bf), 40, 25) == 0
    n = lib.dita_state_cache_bytes_compact(ctypes.byref(bf), 3, 4)
    h = ctypes.c_void_p()
    assert lib.dita_state_cache_init_compact(ctypes.byref(h), ctypes.byref(f32), 5, 3, 4, FAKE_DEV,
                                             1 << 30) == dita.DITA_ERR_DTYPE
    assert lib.dita_state_cache_init_compact(ctypes.byref(h), ctypes.byref(bf), 5, 3, 6, FAKE_DEV,
                                             1 << 30) == dita.DITA_ERR_SHAPE
    assert lib.dita_state_cache_init_compact(ctypes.byref(h), ctypes.byref(bf), 5, 3, 4, FAKE_DEV,
                                             n - 1) == dita.DITA_ERR_SIZE
    assert lib.dita_state_cache_init_compact(ctypes.byref(h), ctypes.byref(bf), 5, 3, 4, FAKE_DEV,
                                             n) == 0
    c = h.value
    fmt = ctypes.c_int()
    for p in range(5):
        assert lib.dita_state_cache_format(c, p, ctypes.byref(fmt)) == 0
        assert fmt.value == dita.DITA_STATE_NONE
        assert lib.dita_state_cache_compact(c, p, None) == dita.DITA_ERR_STATE
        assert lib.dita_state_cache_compact_slot(c, p, None, None, None) == dita.DITA_ERR_STATE
    assert lib.dita_state_cache_compact(c, 5, None) == dita.DITA_ERR_ARG
    assert lib.dita_state_cache_format(c, 0, None) == dita.DITA_ERR_ARG
    on_dev, on_host, free = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.dita_state_cache_residency(c, ctypes.byref(on_dev), ctypes.byref(on_host),
                                          ctypes.byref(free)) == 0
    assert (on_dev.value, on_host.value, free.value) == (0, 0, 3)
    lib.dita_state_cache_free(c)
    # a cache without compact slots has none to give
    u = _cache(bf, 2)
    assert lib.dita_state_cache_compact(u, 0, None) == dita.DITA_ERR_STATE
    lib.dita_state_cache_free(u)
