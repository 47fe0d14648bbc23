"""The allocation-free change statistic (dita_state_change_noalloc) against the
allocating entry point (dita_state_change), through the C ABI: two calls in a
row, the second on a smaller state, each bit for bit (same kernels, same
fixed-order sums), with and without rolling the new state over the previous."""

import numpy as np
import pytest

from gpu_util import say, to_dev, to_host
from oracle.error_planner import state_change
from workloads import round_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("roll", [False, True])
def test_noalloc_change_matches_allocating_entry_point(dev, roll):
    import torch
    import partial_state_reuse_amd as dita
    rng = np.random.default_rng(90)
    cases = [("bf16", (1, 40, 4725, 128)), ("f32", (1, 3, 333, 64))]   # the second is smaller
    out = torch.full((3,), -1.0, dtype=torch.float64, device=dev)
    for dtype, shape in cases:
        say(f"[noalloc] {dtype} {shape} roll={roll}")
        a = rng.standard_normal(shape, dtype=np.float32)
        b = a + np.float32(0.05) * rng.standard_normal(shape, dtype=np.float32)
        if dtype == "bf16":
            a, b = round_bf16(a), round_bf16(b)
        da, db = to_dev(a, dtype, dev), to_dev(b, dtype, dev)
        la = torch.from_numpy(rng.standard_normal(shape[:3]).astype(np.float32)).to(dev)
        lb = torch.zeros_like(la)
        db2, lb2 = db.clone(), lb.clone()
        ref = dita.dita_state_change(da, db, la, lb, roll=roll)
        got = dita.dita_state_change_noalloc(da, db2, out, la, lb2, roll=roll)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert bool((got == ref).all()), (to_host(got), to_host(ref))
        assert bool((db2 == db).all()) and bool((lb2 == lb).all())
        if roll:
            assert bool((db2 == da).all()) and bool((lb2 == la).all())
        expect = state_change(a.astype(np.float64), b.astype(np.float64))
        assert to_host(got)[2] == pytest.approx(expect, rel=1e-12)


def test_noalloc_change_rejects_before_launch(dev):
    import ctypes
    import torch
    import partial_state_reuse_amd as dita
    lib = dita.lib()
    x = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=dev)
    out = torch.zeros(3, dtype=torch.float64, device=dev)
    shape = dita.make_shape(x)
    # previous state overlapping the new one; unaligned output; bad roll flag
    assert lib.dita_state_change_noalloc(ctypes.byref(shape), x.data_ptr(), None, x.data_ptr(),
                                         None, 0, out.data_ptr(), None) == dita.DITA_ERR_ARG
    y = torch.zeros_like(x)
    assert lib.dita_state_change_noalloc(ctypes.byref(shape), x.data_ptr(), None, y.data_ptr(),
                                         None, 0, out.data_ptr() + 8, None) == dita.DITA_ERR_ALIGN
    assert lib.dita_state_change_noalloc(ctypes.byref(shape), x.data_ptr(), None, y.data_ptr(),
                                         None, 2, out.data_ptr(), None) == dita.DITA_ERR_ARG
