"""Key-split attention launches against the fp64 oracle.

When a launch's 512-row tiles do not fill the last round of the compute
units, the tiles of that round are computed in pieces along the key axis by
several workgroups and combined by their LSEs (the state composition applied
to key sub-ranges of one partition).  Every case first asks the library for
its launch layout and checks that the split is really taken, then compares the
result with the oracle, which computes each state in one piece over all keys.
Also: bit-identical repeats, two streams at once, a captured launch, and a
grouped step whose fresh blocks are split.
"""

import numpy as np
import pytest

from gpu_util import assert_state_close, say, to_dev, to_host
from oracle import partial_state
from workloads import round_bf16

pytestmark = pytest.mark.gpu


def _inputs(rng, H, nq, nk, D, scale=1.5, vscale=0.5):
    q = round_bf16(rng.standard_normal((1, H, nq, D)).astype(np.float32) * np.float32(scale))
    k = round_bf16(rng.standard_normal((1, H, nk, D)).astype(np.float32) * np.float32(scale))
    v = round_bf16(rng.standard_normal((1, H, nk, D)).astype(np.float32) * np.float32(vscale))
    return q, k, v


def _layout(H, nq, D, n_blocks, nk):
    import partial_state_reuse_amd as dita
    return dita.dita_attn_launch_info(1, H, nq, D, n_blocks, nk)


def _check_layout(lay, H, nq, n_blocks):
    """The layout's own bookkeeping: the remainder of the 512-row tiles is split."""
    n = -(-nq // 512) * H * n_blocks
    cus = lay["compute_units"]
    assert lay["split_units"] > 0, lay
    assert lay["big_tiles"] == -(-nq // 512) and lay["small_tiles"] == 0, lay
    assert lay["split_tiles"] == n % cus, lay
    assert lay["split_units"] > lay["split_tiles"], lay
    assert lay["workgroups"] == n - lay["split_tiles"] + lay["split_units"], lay
    assert 2 <= lay["max_pieces"] <= 8, lay
    assert 0 < lay["scratch_bytes"] <= lay["scratch_allocated"], lay


# (H, nq, nk, D): several pieces per tile; ragged query rows and a last key
# tile of one key; D = 64 (64-key tiles, a ragged last one); one query tile in
# six pieces; a very long key range.
SPLIT_CASES = [(3, 1000, 3000, 128), (2, 517, 2049, 128), (2, 700, 4001, 64),
               (1, 40, 20000, 128), (1, 333, 70001, 64)]


@pytest.mark.parametrize("H,nq,nk,D", SPLIT_CASES)
def test_split_partial_matches_oracle(dev, H, nq, nk, D):
    import partial_state_reuse_amd as dita
    lay = _layout(H, nq, D, 1, nk)
    say(f"[split] partial H={H} nq={nq} nk={nk} D={D} layout={lay}")
    _check_layout(lay, H, nq, 1)
    rng = np.random.default_rng(H * 1009 + nq * 7 + nk + D)
    q, k, v = _inputs(rng, H, nq, nk, D)
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev))
    o_ref, lse_ref = partial_state(q, k, v)
    eo, el = assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "split partial")
    say(f"  O err {eo:.2e}  LSE err {el:.2e}")


def test_split_with_batches_matches_oracle(dev):
    """B = 2: tiles decode through B * H (heads of both batch entries)."""
    import partial_state_reuse_amd as dita
    B, H, nq, nk, D = 2, 3, 600, 3001, 128
    lay = dita.dita_attn_launch_info(B, H, nq, D, 1, nk)
    say(f"[split] batches layout={lay}")
    _check_layout(lay, B * H, nq, 1)
    rng = np.random.default_rng(29)
    q = round_bf16(rng.standard_normal((B, H, nq, D)).astype(np.float32) * np.float32(1.5))
    k = round_bf16(rng.standard_normal((B, H, nk, D)).astype(np.float32) * np.float32(1.5))
    v = round_bf16(rng.standard_normal((B, H, nk, D)).astype(np.float32) * np.float32(0.5))
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev))
    o_ref, lse_ref = partial_state(q, k, v)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "split, B = 2")


def test_split_peaked_scores_matches_oracle(dev):
    """Keys sorted by score, so the running max moves in every piece and the
    pieces' maxima differ widely: the combination's weights span many octaves."""
    import partial_state_reuse_amd as dita
    H, nq, nk, D = 2, 600, 2500, 128
    lay = _layout(H, nq, D, 1, nk)
    say(f"[split] peaked layout={lay}")
    _check_layout(lay, H, nq, 1)
    rng = np.random.default_rng(31)
    q, k, v = _inputs(rng, H, nq, nk, D, scale=3.0, vscale=0.25)
    order = np.argsort((q[:, :, :1] @ np.swapaxes(k, -1, -2))[..., 0, :], axis=-1)
    k = np.ascontiguousarray(np.take_along_axis(k, order[..., None], axis=2))
    v = np.ascontiguousarray(np.take_along_axis(v, order[..., None], axis=2))
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev), scale=0.3)
    o_ref, lse_ref = partial_state(q, k, v, scale=0.3)
    assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "split, peaked")


def test_split_after_whole_rounds_matches_oracle(dev):
    """More tiles than compute units: whole-tile rounds first, then the split
    remainder.  Heads 0 and the last six (which hold the remainder tiles, in
    linear order) are compared in full."""
    import partial_state_reuse_amd as dita
    H, nq, nk, D = 30, 4725, 2000, 128
    lay = _layout(H, nq, D, 1, nk)
    say(f"[split] whole rounds + split layout={lay}")
    _check_layout(lay, H, nq, 1)
    rng = np.random.default_rng(37)
    q, k, v = _inputs(rng, H, nq, nk, D)
    o, lse = dita.dita_attn_partial(to_dev(q, "bf16", dev), to_dev(k, "bf16", dev),
                                    to_dev(v, "bf16", dev))
    o_h, l_h = to_host(o), to_host(lse)
    tiles = -(-nq // 512)
    first_split_head = (tiles * H - lay["split_tiles"]) // tiles
    heads = sorted({0} | set(range(min(first_split_head, H - 6), H)))
    for h in heads:
        sl = slice(h, h + 1)
        o_ref, lse_ref = partial_state(q[:, sl], k[:, sl], v[:, sl])
        assert_state_close(o_h[:, sl], l_h[:, sl], o_ref, lse_ref, "bf16", f"head {h}")


def test_split_is_bitwise_deterministic(dev):
    """The pieces of a tile finish in no fixed order; the combination reads them
    all from the scratch in key order, so repeats agree bit for bit."""
    import torch
    import partial_state_reuse_amd as dita
    H, nq, nk, D = 4, 1100, 4725, 128
    _check_layout(_layout(H, nq, D, 1, nk), H, nq, 1)
    rng = np.random.default_rng(41)
    q, k, v = _inputs(rng, H, nq, nk, D)
    tq, tk, tv = to_dev(q, "bf16", dev), to_dev(k, "bf16", dev), to_dev(v, "bf16", dev)
    o0, l0 = dita.dita_attn_partial(tq, tk, tv)
    for r in range(4):
        junk = torch.randn(1 << 20, device=dev).sum()
        o1, l1 = dita.dita_attn_partial(tq, tk, tv)
        torch.cuda.synchronize()
        assert bool((o1 == o0).all()) and bool((l1 == l0).all()), f"repeat {r}"
        del junk


def test_split_on_two_streams(dev):
    """Two split launches issued on two streams while the first is still queued:
    they share the library's scratch, which orders them; each result equals the
    one computed alone, bit for bit."""
    import torch
    import partial_state_reuse_amd as dita
    H, nq, nk, D = 3, 1000, 3000, 128
    rng = np.random.default_rng(43)
    qa, ka, va = _inputs(rng, H, nq, nk, D)
    qb, kb, vb = _inputs(rng, H, nq, nk, D)
    da = [to_dev(x, "bf16", dev) for x in (qa, ka, va)]
    db = [to_dev(x, "bf16", dev) for x in (qb, kb, vb)]
    ra = dita.dita_attn_partial(*da)
    rb = dita.dita_attn_partial(*db)
    torch.cuda.synchronize()
    oa, la = torch.empty_like(da[0]), torch.empty((1, H, nq), dtype=torch.float32, device=dev)
    ob, lb = torch.empty_like(db[0]), torch.empty((1, H, nq), dtype=torch.float32, device=dev)
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    say("[split] two streams")
    with torch.cuda.stream(s1):
        torch.cuda._sleep(20_000_000)          # keep s1's launch queued while s2 issues
        dita.dita_attn_partial(*da, o=oa, lse=la)
    with torch.cuda.stream(s2):
        dita.dita_attn_partial(*db, o=ob, lse=lb)
    torch.cuda.current_stream().wait_stream(s1)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    assert bool((oa == ra[0]).all()) and bool((la == ra[1]).all())
    assert bool((ob == rb[0]).all()) and bool((lb == rb[1]).all())
    o_ref, lse_ref = partial_state(qb, kb, vb)
    assert_state_close(to_host(ob), to_host(lb), o_ref, lse_ref, "bf16", "stream 2")


def test_split_in_captured_graph(dev):
    """A split launch captured in a HIP graph (after an eager call made the
    scratch) replays bit for bit, with other eager work between the replays,
    larger split launches among it."""
    import torch
    import partial_state_reuse_amd as dita
    H, nq, nk, D = 2, 517, 2049, 128
    rng = np.random.default_rng(47)
    q, k, v = _inputs(rng, H, nq, nk, D)
    tq, tk, tv = to_dev(q, "bf16", dev), to_dev(k, "bf16", dev), to_dev(v, "bf16", dev)
    o_ref, l_ref = dita.dita_attn_partial(tq, tk, tv)
    torch.cuda.synchronize()
    o = torch.zeros_like(o_ref)
    lse = torch.zeros_like(l_ref)
    say("[split] capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dita.dita_attn_partial(tq, tk, tv, o=o, lse=lse)
    # between replays: other work, and eager split launches with more units
    # than the captured one (the scratch must keep its address for the graph)
    big = _inputs(rng, 6, 1000, 3000, D)
    bq, bk, bv = (to_dev(x, "bf16", dev) for x in big)
    assert _layout(6, 1000, D, 1, 3000)["split_units"] > _layout(H, nq, D, 1, nk)["split_units"]
    for r in range(4):
        o.zero_()
        lse.fill_(-1.0)
        junk = torch.randn(1 << 20, device=dev).sum()
        dita.dita_attn_partial(bq, bk, bv)
        g.replay()
        torch.cuda.synchronize()
        assert bool((o == o_ref).all()) and bool((lse == l_ref).all()), f"replay {r}"
        del junk


def test_step_with_split_fresh_blocks(dev):
    """A rank-step whose three fresh blocks (equal lengths) share one split
    launch: the fresh states and the merged output against the oracle."""
    import torch
    import partial_state_reuse_amd as dita
    from oracle import StateCache as OracleCache
    from oracle import attn_step as oracle_step
    H, nq, nk, D, P = 8, 1100, 1500, 128, 6
    lay = _layout(H, nq, D, 3, nk)
    say(f"[split] step, 3 fresh blocks, layout={lay}")
    _check_layout(lay, H, nq, 3)
    rng = np.random.default_rng(53)
    q = round_bf16(rng.standard_normal((1, H, nq, D)).astype(np.float32) * 1.5)
    ks = [round_bf16(rng.standard_normal((1, H, nk, D)).astype(np.float32) * 1.5) for _ in range(P)]
    vs = [round_bf16(rng.standard_normal((1, H, nk, D)).astype(np.float32) * 0.5) for _ in range(P)]
    qd = to_dev(q, "bf16", dev)
    kd = [to_dev(x, "bf16", dev) for x in ks]
    vd = [to_dev(x, "bf16", dev) for x in vs]
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    ref = OracleCache(P)
    for step, mask in enumerate([np.zeros(P, np.uint8), np.array([1, 0, 1, 0, 1, 0], np.uint8)]):
        o, lse, info = dita.dita_attn_step(cache, qd, kd, vd, mask, step)
        o_ref, lse_ref, _ = oracle_step(ref, q, ks, vs, mask, step)
        assert_state_close(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", f"step {step}")
        for p in range(P):
            so, sl = cache.slot(p)
            ro, rl = ref.slots[p]
            assert_state_close(to_host(so), to_host(sl), ro, rl, "bf16", f"step {step} state {p}")
    assert info.n_fresh == 3
