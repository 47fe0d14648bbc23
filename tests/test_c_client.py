"""The library's C ABI used from plain C (tests/c/dita_c_client.c), no Python in
between: host-only checks on the CPU, and on the GPU a three-step schedule whose
outputs are compared with the fp64 oracle."""

import os
import subprocess

import numpy as np
import pytest

from oracle import StateCache as OracleCache
from oracle import attn_step as oracle_step
from workloads import round_bf16

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c", "dita_c_client")


def _client():
    if not os.path.exists(CLIENT):
        import importlib.util
        spec = importlib.util.spec_from_file_location("_client_build", os.path.join(HERE, "c", "build_client.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return CLIENT


def test_c_client_host_checks():
    r = subprocess.run([_client(), "check"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=60)
    assert r.returncode == 0, r.stdout
    assert "check ok" in r.stdout


def _bf16_bytes(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16).tobytes()


def _from_bf16(path, shape):
    u = np.fromfile(path, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64).reshape(shape)


@pytest.mark.gpu
def test_c_client_steps_match_oracle(tmp_path):
    rng = np.random.default_rng(40)
    B, H, Nq, D = 1, 3, 200, 128
    nk = [130, 77, 256, 190]
    P = len(nk)
    q = round_bf16(rng.standard_normal((B, H, Nq, D)) * 1.2)
    ks = [round_bf16(rng.standard_normal((B, H, n, D)) * 1.2) for n in nk]
    vs = [round_bf16(rng.standard_normal((B, H, n, D)) * 0.5) for n in nk]
    masks = [np.zeros(P, np.uint8), np.array([0, 1, 0, 1], np.uint8), np.ones(P, np.uint8)]
    d = str(tmp_path)
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"{B} {H} {D} {Nq} {P} {len(masks)} 1\n")
    with open(os.path.join(d, "nk.txt"), "w") as f:
        f.write(" ".join(map(str, nk)) + "\n")
    open(os.path.join(d, "q.bin"), "wb").write(_bf16_bytes(q))
    for p in range(P):
        open(os.path.join(d, f"k{p}.bin"), "wb").write(_bf16_bytes(ks[p]))
        open(os.path.join(d, f"v{p}.bin"), "wb").write(_bf16_bytes(vs[p]))
    for s, m in enumerate(masks):
        open(os.path.join(d, f"mask{s}.bin"), "wb").write(m.tobytes())
    print("[c client] run", d, flush=True)
    r = subprocess.run([_client(), "run", d], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    ref = OracleCache(P)
    prev = None
    for s, m in enumerate(masks):
        o_ref, lse_ref, nf = oracle_step(ref, q, ks, vs, m, s)
        o = _from_bf16(os.path.join(d, f"o{s}.bin"), (B, H, Nq, D))
        lse = np.fromfile(os.path.join(d, f"lse{s}.bin"), dtype=np.float32).astype(np.float64)
        lse = lse.reshape(B, H, Nq)
        assert np.max(np.abs(o - o_ref)) <= 1e-2 and np.max(np.abs(lse - lse_ref)) <= 1e-3, s
        n_fresh, n_reused = map(int, open(os.path.join(d, f"info{s}.txt")).read().split())
        assert (n_fresh, n_reused) == (nf, P - nf)
        if s == 2:   # all reuse: the previous step's output, bit for bit
            assert np.array_equal(o, prev[0]) and np.array_equal(lse, prev[1])
        prev = (o, lse)
