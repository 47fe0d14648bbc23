"""Helpers shared by the GPU parity tests (not a test module)."""

from __future__ import annotations

import sys

import numpy as np

# Acceptance tolerances (max-abs): fp32 1e-5 on O and LSE; bf16 1e-2 on O, 1e-3 on LSE.
TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str, dev):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)      # exact: the values are bf16-representable
    return t.to(dev)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        raise AssertionError(f"shape {a.shape} vs {b.shape}")
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def assert_state_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str = ""):
    to, tl = TOL[dtype]
    eo, el = max_abs(o_gpu, o_ref), max_abs(lse_gpu, lse_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    assert eo <= to, f"{what}: O max-abs {eo:.3e} > {to:.0e}"
    assert el <= tl, f"{what}: LSE max-abs {el:.3e} > {tl:.0e}"
    return eo, el
