"""A rank-step captured in a HIP graph (through torch.cuda.graph) and replayed:
every replay must reproduce the eagerly computed step bit for bit, with other
eager work and synchronisations between the replays.  Capture records the
launches of one step with its mask and slot assignment fixed, which is how a
caller would replay a launch-bound step of a fixed schedule."""

import numpy as np
import pytest

from gpu_util import say, to_dev
from workloads import round_bf16

pytestmark = pytest.mark.gpu


def test_captured_step_replays_bitwise(dev):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(50)
    P, H, nq, D = 5, 4, 333, 128
    lengths = [256, 190, 300, 77, 128]
    q = round_bf16(rng.standard_normal((1, H, nq, D)) * 1.2)
    ks = [round_bf16(rng.standard_normal((1, H, n, D)) * 1.2) for n in lengths]
    vs = [round_bf16(rng.standard_normal((1, H, n, D)) * 0.5) for n in lengths]
    qd = to_dev(q, "bf16", dev)
    kd = [to_dev(x, "bf16", dev) for x in ks]
    vd = [to_dev(x, "bf16", dev) for x in vs]
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P, device=dev)
    dita.dita_attn_step(cache, qd, kd, vd, np.zeros(P, np.uint8), 0)       # fill, eager
    mask = np.array([0, 0, 1, 1, 1], np.uint8)
    o = torch.empty((1, H, nq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, H, nq), dtype=torch.float32, device=dev)
    dita.dita_attn_step(cache, qd, kd, vd, mask, 1, o=o, lse=lse)           # eager reference
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    say("[graph] capture")
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o.zero_()
        lse.zero_()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dita.dita_attn_step(cache, qd, kd, vd, mask, 1, o=o, lse=lse)
    for r in range(4):
        o.zero_()
        lse.fill_(-1.0)
        junk = torch.randn(1 << 20, device=dev).sum()     # other eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert bool((o == o_ref).all()) and bool((lse == lse_ref).all()), f"replay {r}"
        del junk
