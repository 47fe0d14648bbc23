"""GPU parity of the individual entry points against the fp64 oracle.

Sizes span several query and key tiles with ragged tails on both axes, both
head dims, both dtypes.  Inputs are seeded; bf16 inputs are rounded once and
the oracle consumes exactly those values.
"""

import numpy as np
import pytest

from gpu_util import TOL, assert_state_close, max_abs, say, to_dev, to_host
from oracle import merge_states, partial_state
from workloads import round_bf16

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (5, 1), (77, 63), (128, 64), (129, 65), (300, 257), (256, 1000), (1, 700)]


def _inputs(rng, B, H, nq, nk, D, dtype, scale=1.0):
    # V ~ 0.5 N(0,1), the value scale of the video-DiT workloads: the absolute bf16
    # bound on O (1e-2) presumes |O| below ~2, where bf16's half-ulp is <= 0.0039.
    q = rng.standard_normal((B, H, nq, D)).astype(np.float32) * np.float32(scale)
    k = rng.standard_normal((B, H, nk, D)).astype(np.float32) * np.float32(scale)
    v = rng.standard_normal((B, H, nk, D)).astype(np.float32) * np.float32(0.5)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_attn_partial_matches_oracle(dev, dtype, D, nq, nk):
    import partial_state_reuse_amd as dita
    say(f"attn_partial dtype={dtype} D={D} nq={nq} nk={nk}")
    rng = np.random.default_rng(nq * 7919 + nk * 31 + D)
    q, k, v = _inputs(rng, 1, 2, nq, nk, D, dtype, scale=1.5)
    o, lse = dita.dita_attn_partial(to_dev(q, dtype, dev), to_dev(k, dtype, dev), to_dev(v, dtype, dev))
    o_ref, lse_ref = partial_state(q, k, v)
    eo, el = assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "attn_partial")
    say(f"  O err {eo:.2e}  LSE err {el:.2e}")


@pytest.mark.parametrize("D", [64, 128])
def test_attn_partial_large_scores_and_batches(dev, D):
    """Scores spanning ~+-60 (exercises the lazy rescale) with B=2, H=3, explicit scale."""
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(5 + D)
    q, k, v = _inputs(rng, 2, 3, 200, 900, D, "bf16", scale=3.0)
    # sort keys so that later tiles hold larger scores and the running max moves often
    order = np.argsort((q[:, :, :1] @ np.swapaxes(k, -1, -2))[..., 0, :], axis=-1)
    k = np.take_along_axis(k, order[..., None], axis=2)
    v = np.take_along_axis(v, order[..., None], axis=2)
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev), scale=0.25)
    o_ref, lse_ref = partial_state(q, k, v, scale=0.25)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "large scores")


def test_attn_partial_is_deterministic(dev):
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(9)
    q, k, v = _inputs(rng, 1, 4, 333, 777, 128, "bf16")
    tq, tk, tv = to_dev(q, "bf16", dev), to_dev(k, "bf16", dev), to_dev(v, "bf16", dev)
    o1, l1 = dita.dita_attn_partial(tq, tk, tv)
    o2, l2 = dita.dita_attn_partial(tq, tk, tv)
    assert bool((o1 == o2).all()) and bool((l1 == l2).all())


def _states(rng, P, B, H, nq, D, dtype, neg_inf_slot=None):
    os_, ls = [], []
    for p in range(P):
        o = rng.standard_normal((B, H, nq, D)).astype(np.float32)
        l = (3.0 * rng.standard_normal((B, H, nq)) + 5.0).astype(np.float32)
        if dtype == "bf16":
            o = round_bf16(o)
        if p == neg_inf_slot:
            l[:] = -np.inf
        os_.append(o)
        ls.append(l)
    return os_, ls


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 9, 16, 64])
def test_state_merge_matches_oracle(dev, dtype, D, P):
    import partial_state_reuse_amd as dita
    say(f"merge dtype={dtype} D={D} P={P}")
    rng = np.random.default_rng(P * 100 + D)
    os_, ls = _states(rng, P, 1, 3, 37, D, dtype, neg_inf_slot=1 if P > 2 else None)
    o, lse = dita.dita_state_merge([to_dev(x, dtype, dev) for x in os_],
                                   [to_dev(x, "f32", dev) for x in ls])
    o_ref, lse_ref = merge_states(list(zip(os_, ls)))
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "merge")


def test_state_merge_all_neutral_rows(dev):
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(3)
    os_, ls = _states(rng, 3, 1, 1, 8, 64, "f32")
    for l in ls:
        l[0, 0, :4] = -np.inf
    o, lse = dita.dita_state_merge([to_dev(x, "f32", dev) for x in os_],
                                   [to_dev(x, "f32", dev) for x in ls])
    o, lse = to_host(o), to_host(lse)
    assert np.all(o[0, 0, :4] == 0) and np.all(np.isneginf(lse[0, 0, :4]))
    o_ref, lse_ref = merge_states(list(zip(os_, ls)))
    assert max_abs(o[0, 0, 4:], o_ref[0, 0, 4:]) <= 1e-5


def test_state_merge_single_state_is_identity_bitwise(dev):
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(4)
    os_, ls = _states(rng, 1, 1, 2, 50, 128, "bf16")
    o, lse = dita.dita_state_merge([to_dev(os_[0], "bf16", dev)], [to_dev(ls[0], "f32", dev)])
    assert np.array_equal(to_host(o), os_[0].astype(np.float64))
    assert np.array_equal(to_host(lse), ls[0].astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_store_load_roundtrip_bitwise(dev, dtype):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(6)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = dita.StateCache(1, 2, 77, 128, tdt, P=3, device=dev)
    os_, ls = _states(rng, 3, 1, 2, 77, 128, dtype)
    for p in range(3):
        cache.store(p, to_dev(os_[p], dtype, dev), to_dev(ls[p], "f32", dev), step=10 + p)
    for p in (2, 0, 1):
        o, l = cache.load(p)
        assert np.array_equal(to_host(o), os_[p].astype(np.float64))
        assert np.array_equal(to_host(l), ls[p].astype(np.float64))
        assert cache.info(p) == (True, 10 + p)
        so, sl = cache.slot(p)
        assert bool((so == o).all()) and bool((sl == l).all())
    cache.invalidate(1)
    assert cache.info(1) == (False, -1)
    with pytest.raises(dita.DitaError):
        cache.load(1)


@pytest.mark.parametrize("D", [64, 128])
def test_attn_partial_peaked_scores_all_waves(dev, D):
    """Peaked scores (exact max / rescale path after the first tile) on more than
    512 queries, so every wave of a workgroup and a second query tile take it."""
    import partial_state_reuse_amd as dita
    say(f"attn_partial peaked scores D={D}")
    rng = np.random.default_rng(11 + D)
    q, k, v = _inputs(rng, 1, 2, 700, 1100, D, "bf16", scale=3.0)
    # score std ~9: one key dominates each row, so |O| reaches max |v|; V at
    # 0.25 N(0,1) keeps |O| below ~1.5, where the absolute bf16 bound holds
    v = round_bf16(v * np.float32(0.5))
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev))
    o_ref, lse_ref = partial_state(q, k, v)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "peaked scores")


def test_attn_partial_largest_key_slice(dev):
    """The largest partition one head may hold: nk * D * 2 bytes just under 2^31
    (the kernel addresses a head's K and V through 32-bit buffer records).  Keys
    near the very end carry the largest scores, so a misread tail would show."""
    import partial_state_reuse_amd as dita
    D, nq = 128, 40
    nk = (1 << 31) // (D * 2) - 1
    say(f"attn_partial largest key slice nk={nk}")
    rng = np.random.default_rng(12)
    q = round_bf16(rng.standard_normal((1, 1, nq, D), dtype=np.float32))
    blk = 1 << 20                                   # a random block of keys, repeated
    reps = -(-nk // blk)
    k = np.tile(round_bf16(rng.standard_normal((1, 1, blk, D), dtype=np.float32)), (1, 1, reps, 1))[:, :, :nk]
    v = np.tile(round_bf16(rng.standard_normal((1, 1, blk, D), dtype=np.float32) * np.float32(0.5)),
                (1, 1, reps, 1))[:, :, :nk]
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    k[0, 0, nk - nq:] = round_bf16(3.0 * q[0, 0])   # key nk-nq+i aligns with query i
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev))
    # the oracle over key chunks, composed exactly (merge of partial states)
    o_ref, lse_ref = merge_states([partial_state(q, k[:, :, a:a + blk], v[:, :, a:a + blk])
                                   for a in range(0, nk, blk)])
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "largest key slice")
    lse_host = to_host(lse)[0, 0]
    assert np.all(lse_host > 20.0)                  # the planted tail keys dominate every row


def test_attn_partial_most_heads(dev):
    """B * H = 65535, the most (batch, head) pairs a launch takes."""
    import partial_state_reuse_amd as dita
    say("attn_partial B*H = 65535")
    rng = np.random.default_rng(13)
    q, k, v = _inputs(rng, 3, 21845, 33, 17, 64, "bf16", scale=1.5)
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev))
    o_ref, lse_ref = partial_state(q, k, v)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "B*H = 65535")


def test_step_with_most_partitions(dev):
    """A rank-step over 64 partitions (the most a cache holds), ragged lengths, then
    a mixed reuse step."""
    import torch
    import partial_state_reuse_amd as dita
    from oracle import StateCache as OracleCache
    from oracle import attn_step as oracle_step
    say("attn_step P = 64")
    rng = np.random.default_rng(14)
    P, H, nq, D = 64, 2, 70, 64
    lengths = [int(x) for x in rng.integers(1, 90, P)]
    q = round_bf16(rng.standard_normal((1, H, nq, D), dtype=np.float32) * np.float32(1.2))
    ks = [round_bf16(rng.standard_normal((1, H, n, D), dtype=np.float32) * np.float32(1.2)) for n in lengths]
    vs = [round_bf16(rng.standard_normal((1, H, n, D), dtype=np.float32) * np.float32(0.5)) for n in lengths]
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    ref = OracleCache(P)
    qd = to_dev(q, "bf16", dev)
    kd = [to_dev(x, "bf16", dev) for x in ks]
    vd = [to_dev(x, "bf16", dev) for x in vs]
    for s, mask in enumerate([np.zeros(P, np.uint8), (rng.random(P) < 0.5).astype(np.uint8)]):
        o, lse, info = dita.dita_attn_step(cache, qd, kd, vd, mask, s)
        o_ref, lse_ref, nf = oracle_step(ref, q, ks, vs, mask, s)
        assert info.n_fresh == nf
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", f"P=64 step {s}")


def test_step_with_one_partition(dev):
    """P = 1: the step's merge is the identity on the one state (bit for bit), and
    an all-reuse step returns the same output again."""
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(15)
    q, k, v = _inputs(rng, 1, 3, 150, 333, 128, "bf16", scale=1.5)
    qd, kd, vd = to_dev(q, "bf16", dev), to_dev(k, "bf16", dev), to_dev(v, "bf16", dev)
    cache = dita.StateCache(1, 3, 150, 128, torch.bfloat16, 1, device=dev)
    o, lse, info = dita.dita_attn_step(cache, qd, [kd], [vd], np.zeros(1, np.uint8), 0)
    assert info.n_fresh == 1 and info.merge_sources == 1
    so, sl = cache.slot(0)
    assert bool((o == so).all()) and bool((lse == sl).all())
    o_ref, lse_ref = partial_state(q, k, v)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "P = 1")
    o2, l2, info = dita.dita_attn_step(cache, qd, [None], [None], np.ones(1, np.uint8), 1)
    assert info.n_fresh == 0 and bool((o2 == o).all()) and bool((l2 == lse).all())


@pytest.mark.parametrize("D", [64, 128])
def test_grouped_launch_with_256_row_tiles(dev, D):
    """A grouped launch large enough (300 (head, block) pairs, more than a round of
    the compute units) that the rows past the last whole 512-row tile go into
    256-row tiles dispatched at the end: every head, every row against the oracle."""
    import torch
    import partial_state_reuse_amd as dita
    from oracle import StateCache as OracleCache
    from oracle import attn_step as oracle_step
    rng = np.random.default_rng(70 + D)
    H, nq = 60, 600                          # 600 = 512 + 88 rows
    lengths = [200, 333, 64, 517, 129]
    P = len(lengths)
    q = round_bf16(rng.standard_normal((1, H, nq, D)).astype(np.float32) * 1.5)
    ks = [round_bf16(rng.standard_normal((1, H, n, D)).astype(np.float32) * 1.5) for n in lengths]
    # V at 0.35 N(0,1): with these peaked scores |O| approaches single value rows, and the
    # absolute 1e-2 bound presumes |O| < 2 (bf16 spacing above 2 is 1/64)
    vs = [round_bf16(rng.standard_normal((1, H, n, D)).astype(np.float32) * 0.35) for n in lengths]
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    ref = OracleCache(P)
    fresh = np.zeros(P, np.uint8)
    o, lse, info = dita.dita_attn_step(cache, to_dev(q, "bf16", dev), [to_dev(x, "bf16", dev) for x in ks],
                                       [to_dev(x, "bf16", dev) for x in vs], fresh, 0)
    o_ref, lse_ref, _ = oracle_step(ref, q, ks, vs, fresh, 0)
    assert info.n_fresh == P
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "grouped, 256-row tiles")
    for p in range(P):
        so, sl = cache.slot(p)
        ro, rl = ref.slots[p]
        assert_state_close(to_host(so), to_host(sl), ro, rl, "bf16", f"fresh state {p}")


# (H, nq, P, nk, D): tails of 88 or 52 rows; pairs even (320) and odd (287);
# D = 64 with four whole 512-row tiles before the tail.
# (H, nq, P, nk, D) launches that the planner lays out staged on a 256-CU
# device: every 512-row tile first, then every 256-row tile, with some pairs
# holding one 512-row tile fewer and two 256-row tiles more (or, last case,
# 256-row tiles only).
# (B, H, nq, P, nk, D); the B = 2 case decodes pairs through B * H.
STAGED_CASES = [(1, 24, 1100, 6, 300, 128), (1, 41, 1300, 5, 300, 64), (1, 12, 1800, 8, 300, 64),
                (1, 8, 1000, 1, 700, 128), (2, 12, 1100, 6, 300, 128)]


@pytest.mark.parametrize("B,H,nq,P,nk,D", STAGED_CASES)
def test_grouped_launch_with_staged_tiles(dev, B, H, nq, P, nk, D):
    """A grouped launch in the staged layout: the library's layout says so, its
    tile counts add up to the grid, and every head and row of the step output
    and of every fresh state matches the oracle."""
    import torch
    import partial_state_reuse_amd as dita
    from gpu_util import HeadChunkedOracle
    lay = dita.dita_attn_launch_info(B, H, nq, D, P, nk)
    say(f"staged tiles B={B} H={H} nq={nq} P={P} nk={nk} D={D} layout={lay}")
    if lay["compute_units"] != 256:
        pytest.skip("layout chosen for a 256-CU device")
    pairs = B * H * P
    a = lay["staged_pairs"]
    assert 0 <= a <= pairs and lay["split_units"] == 0 and lay["dual_tails"] == 0, lay
    n_big = a * lay["big_tiles"] + (pairs - a) * (lay["big_tiles"] - 1)
    n_small = a * lay["small_tiles"] + (pairs - a) * lay["small_tiles_b"]
    assert n_small > 0 and lay["workgroups"] == n_big + n_small, lay
    rng = np.random.default_rng(B * 1009 + H * 37 + nq + P + D)
    q = round_bf16(rng.standard_normal((B, H, nq, D)).astype(np.float32) * 1.5)
    ks = [round_bf16(rng.standard_normal((B, H, nk, D)).astype(np.float32) * 1.5) for _ in range(P)]
    vs = [round_bf16(rng.standard_normal((B, H, nk, D)).astype(np.float32) * 0.35) for _ in range(P)]
    cache = dita.StateCache(B, H, nq, D, torch.bfloat16, P, device=dev)
    fresh = np.zeros(P, np.uint8)
    o, lse, info = dita.dita_attn_step(cache, to_dev(q, "bf16", dev), [to_dev(x, "bf16", dev) for x in ks],
                                       [to_dev(x, "bf16", dev) for x in vs], fresh, 0)
    assert info.n_fresh == P
    o_h, l_h = to_host(o), to_host(lse)
    slots = [tuple(to_host(t) for t in cache.slot(p)) for p in range(P)]
    for b in range(B):  # the head-chunked oracle takes one batch entry at a time
        ref = HeadChunkedOracle(P, H, chunk=max(1, H // 16))
        o_ref, lse_ref, _ = ref.step(q[b:b + 1], [x[b:b + 1] for x in ks], [x[b:b + 1] for x in vs],
                                     fresh, 0)
        assert_state_close(o_h[b:b + 1], l_h[b:b + 1], o_ref, lse_ref, "bf16",
                           f"staged tiles, output, batch {b}")
        for p in range(P):
            ro, rl = ref.slot(p)
            assert_state_close(slots[p][0][b:b + 1], slots[p][1][b:b + 1], ro, rl, "bf16",
                               f"staged tiles, state {p}, batch {b}")

DUAL_CASES = [(40, 600, 8, 700, 128), (41, 600, 7, 700, 128), (40, 2100, 8, 700, 64)]


@pytest.mark.parametrize("H,nq,P,nk,D", DUAL_CASES)
def test_grouped_launch_with_dual_tail_tiles(dev, H, nq, P, nk, D):
    """A grouped launch whose tail rows (at most 128 per (head, block)) go two
    pairs per 256-row workgroup, each wave group with its own K/V ring: the
    library's layout says so, and every head and row of the step output and of
    every fresh state matches the oracle (an odd pair count leaves the last
    workgroup's second half without rows)."""
    import torch
    import partial_state_reuse_amd as dita
    from gpu_util import HeadChunkedOracle
    lay = dita.dita_attn_launch_info(1, H, nq, D, P, nk)
    say(f"dual tails H={H} nq={nq} P={P} nk={nk} D={D} layout={lay}")
    assert lay["dual_tails"] == 1 and lay["small_tiles"] == 1 and lay["split_units"] == 0, lay
    pairs = H * P
    assert lay["workgroups"] == lay["big_tiles"] * pairs + (pairs + 1) // 2, lay
    rng = np.random.default_rng(H * 31 + nq + P + D)
    q = round_bf16(rng.standard_normal((1, H, nq, D)).astype(np.float32) * 1.5)
    ks = [round_bf16(rng.standard_normal((1, H, nk, D)).astype(np.float32) * 1.5) for _ in range(P)]
    vs = [round_bf16(rng.standard_normal((1, H, nk, D)).astype(np.float32) * 0.35) for _ in range(P)]
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    fresh = np.zeros(P, np.uint8)
    o, lse, info = dita.dita_attn_step(cache, to_dev(q, "bf16", dev), [to_dev(x, "bf16", dev) for x in ks],
                                       [to_dev(x, "bf16", dev) for x in vs], fresh, 0)
    assert info.n_fresh == P
    ref = HeadChunkedOracle(P, H, chunk=max(1, H // 16))
    o_ref, lse_ref, _ = ref.step(q, ks, vs, fresh, 0)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "dual tails, output")
    for p in range(P):
        so, sl = cache.slot(p)
        ro, rl = ref.slot(p)
        assert_state_close(to_host(so), to_host(sl), ro, rl, "bf16", f"dual tails, state {p}")
