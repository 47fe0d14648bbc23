"""Benchmark: rank-steps of selective attention-state reuse on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the host mask planner, the grouped fresh partial-attention launch that writes
states into the cache, and the P-way LSE merge, all through the C ABI.

Default workload: 75,600 tokens (21 frames x 45x80 patches), H=40, D=128,
bf16, P=16 context partitions of 4725 tokens; the rank owns partition 0 and
recomputes partitions within distance 2, with a full refresh (anchor) every
5th step.  The K/V of all 10 steps of that schedule are generated up front
and resident in HBM before the timed region; timed step i uses the inputs
and mask of schedule step (warmup + i) mod 10.  Before the warm-up steps,
whole schedule cycles run untimed for --device-warmup seconds (the GPU comes
out of the host-side input generation idle and its clock takes a few hundred
ms of this load to settle); the JSON line reports them as device_warmup.

Prints ONE JSON line:  value = fresh-block attention TFLOP/s over the whole
timed job (fresh-block flops / wall time of the K steps), ms_per_step, the
roofline of the dominant kernel (the fresh-attention launch, timed with HIP
events on its own stream), the merge's bandwidth, and the fp64 CPU oracle
timed on a bounded sample of the same step.

By default (--compose-ahead 1) each step also composes the partitions the
next step will reuse into groups (Dynamic Group Compose; the step's
compose_next option, the largest run in the same pass as its final merge),
so a step's merge reads one state per group; --premerge 1 instead (or also)
merges the reused states on a second stream while the fresh attention runs.

With --trajectory the schedule also runs once from a cold cache beside an
all-fresh reference computed by the same library on the same K/V (every
partition recomputed, which equals full attention): per step the fresh
blocks, the step latency, the max-abs and relative-Frobenius error of the
reused output against the all-fresh one (and its running max), and the
contribution of each partition to the output by distance from the local one
(mean over rows of exp(LSE_p - LSE) at the all-fresh step 0).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--seed S] [--trajectory]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--device-warmup", type=float, default=0.5,
                    help="seconds of whole schedule cycles run (untimed) before the --warmup "
                         "steps: the GPU comes out of the host-side input generation idle, and "
                         "its clock takes a few hundred ms of this load to settle (0: none)")
    ap.add_argument("--workload", default="dit75k_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trajectory", action="store_true",
                    help="also run the whole schedule once from a cold cache beside an all-fresh "
                         "reference and report per-step error, fresh blocks and latency")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--resident-steps", type=int, default=0,
                    help="distinct K/V steps to generate (0: the whole schedule); step s uses "
                         "inputs s mod this, for short profiling runs")
    ap.add_argument("--premerge", type=int, default=0, choices=(0, 1),
                    help="1: merge the reused states on a second stream while the fresh "
                         "attention runs (dita_attn_step_ex)")
    ap.add_argument("--compose-ahead", type=int, default=1, choices=(0, 1),
                    help="1: after each step compose the runs of partitions the next step "
                         "reuses into groups (dita_state_cache_compose_runs); timed")
    ap.add_argument("--planner", choices=("fixed", "error"), default="fixed",
                    help="trajectory only: the workload's fixed schedule, or the error-guided "
                         "group planner (dita_planner_*) fed by the statistics kernels")
    ap.add_argument("--budget", type=float, default=0.004,
                    help="error planner: estimated error allowed to be reused per step")
    ap.add_argument("--group-size", type=int, default=2, help="error planner: partitions per group")
    ap.add_argument("--fresh-weight", type=float, default=0.0,
                    help="error planner: groups holding a partition of at least this "
                         "contribution are always computed (0: off)")
    ap.add_argument("--fixed-radius", type=int, default=-1,
                    help="replace the workload's mask schedule by a fixed distance radius")
    ap.add_argument("--planner-compose", type=int, default=0, choices=(0, 1),
                    help="error planner: compose the runs its next mask reuses after each step")
    ap.add_argument("--planner-anchor", type=int, default=0,
                    help="error planner: anchor period (0: only the cold step)")
    ap.add_argument("--compact", type=int, default=0, choices=(0, 1),
                    help="trajectory only: after each step (and its composition ahead) encode "
                         "every full state the next step reuses into a compact slot (int8 codes, "
                         "per-row scale); reports the bytes held by cached states per step")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the sustained-clock measurement (it polls amd-smi, a separate "
                         "program; skipped by itself under a profiler)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run the library's state-copy kernel over BYTES of O (the "
                         "reference point for HBM byte counters) and exit")
    return ap.parse_args()


def copy_calibration(nbytes: int):
    """Copy a state of known size with the library's copy kernel (cache store), 5 times."""
    import torch
    import partial_state_reuse_amd as dita
    dev = torch.device("cuda:0")
    D, H = 128, 1
    nq = max(1, nbytes // (D * 2))
    cache = dita.StateCache(1, H, nq, D, torch.bfloat16, P=1, device=dev)
    o = torch.zeros((1, H, nq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((1, H, nq), dtype=torch.float32, device=dev)
    for i in range(5):
        cache.store(0, o, lse, step=i)
    torch.cuda.synchronize()
    moved = nq * D * 2 + nq * 4
    print(json.dumps({"copy_calibration": {"launches": 5, "read_bytes_per_launch": moved,
                                           "write_bytes_per_launch": moved}}), flush=True)


def profiled_traffic(workload: str):
    """HBM bytes per launch of the attention and merge kernels from the committed
    rocprofv3 counter summary, each only while its kernel sources are unchanged
    since the counters were taken (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload.replace("_bf16", ""))
    csrc = os.path.join(ROOT, "partial_state_reuse_amd", "csrc")
    if not os.path.exists(path):
        return None, None

    def digest(files):
        h = hashlib.sha256()
        for f in files:
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
        return h.hexdigest()

    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("workload") != workload:
        return None, None
    attn = rec["attn"]["traffic_bytes_per_launch"] \
        if rec["attn"]["sources_sha256"] == digest(["attn_bf16.hip", "dita_kernels.h"]) else None
    merge = rec["merge"]["traffic_bytes_per_launch"] \
        if rec["merge"]["sources_sha256"] == digest(["merge.hip", "dita_kernels.h"]) else None
    return attn, merge


def upload_parts(x: np.ndarray, wl, dev, tdt):
    import torch
    out = []
    for p in range(wl.P):
        a, b = wl.part_range(p)
        out.append(torch.from_numpy(np.ascontiguousarray(x[:, :, a:b])).to(tdt).to(dev))
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [{k: d.get(k) for k in ("internal_api", "num_threads", "version")}
                for d in threadpool_info()]
    except Exception:
        return []


def cpu_baseline(inp, wl, budget_s: float):
    """The fp64 oracle's rank-step, timed as it stands on the host cores: a
    non-anchor step (fresh blocks + P-way merge), its heads spread over a pool of
    worker threads with one BLAS thread each (numpy releases the interpreter lock
    in its matrix products and element-wise kernels; the oracle's exp is
    single-threaded per call, so the parallel width comes from the heads).  Heads
    run in waves of `workers` until about budget_s has passed; one head is also
    timed alone on one core."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import Plan, StateCache, attn_step, plan_mask
    from workloads import split_parts
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    cpus = len(os.sched_getaffinity(0))
    workers = max(1, min(cpus, 16, wl.H))
    plan = Plan(**wl.plan_fields())
    # The first step index whose mask is not all-fresh with every slot filled.
    s = next(i for i in range(1, wl.steps + 1)
             if plan_mask(plan, i % wl.steps, np.ones(wl.P, np.uint8)).any())
    mask = plan_mask(plan, s % wl.steps, np.ones(wl.P, np.uint8))
    k, v = inp.kv(s % wl.steps)
    kp, vp = split_parts(k, wl), split_parts(v, wl)
    block_flops = 4.0 * wl.B * wl.Nq * wl.D * sum(wl.Nk for p in range(wl.P) if mask[p] == 0)

    def setup(h):
        rng = np.random.default_rng(h)
        cache = StateCache(wl.P)
        for p in range(wl.P):   # reused slots: any state of the right shape (untimed)
            cache.store(p, (rng.standard_normal((wl.B, 1, wl.Nq, wl.D)),
                            rng.standard_normal((wl.B, 1, wl.Nq)) + 9.0), 0)
        return cache

    def one(h, cache):
        return attn_step(cache, inp.q[:, h:h + 1], [x[:, h:h + 1] for x in kp],
                         [x[:, h:h + 1] for x in vp], mask, s)

    class _Null:
        def __enter__(self):
            return self

        def __exit__(self, *a):
            return False

    limit = threadpool_limits(1) if threadpool_limits else _Null()
    with limit:
        c0 = setup(0)
        t0 = time.perf_counter()
        one(0, c0)
        single_s = time.perf_counter() - t0
        heads_done, elapsed = 0, 0.0
        with ThreadPoolExecutor(workers) as ex:
            while heads_done < wl.H and elapsed < budget_s:
                wave = list(range(heads_done, min(wl.H, heads_done + workers)))
                caches = [setup(h) for h in wave]
                t0 = time.perf_counter()
                list(ex.map(lambda a: one(*a), zip(wave, caches)))
                elapsed += time.perf_counter() - t0
                heads_done += len(wave)
    host = {"affinity_cpus": cpus, "cpu_model": _cpu_model(), "blas": _blas_info()}
    return {
        "value": block_flops * heads_done / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "host": host,
        "workers": workers,
        "blas_threads_per_worker": 1,
        "ms_per_step": elapsed / heads_done * wl.H * 1e3,
        "single_core": {"heads": 1, "s": single_s, "TFLOPs": block_flops / single_s / 1e12,
                        "ms_per_step": single_s * wl.H * 1e3},
        "sample": (f"fp64 numpy oracle rank-step (schedule step {s % wl.steps}: "
                   f"{int((mask == 0).sum())} fresh blocks + {wl.P}-way merge) on {heads_done} of "
                   f"{wl.H} heads in waves of {workers} worker threads with one BLAS thread each, "
                   f"{elapsed:.1f} s; ms_per_step scaled to all heads"),
    }


def isolated_bandwidth(dita, wl, tdt, dev, stream, q, n_caches: int = 4, reps: int = 3):
    """Merge and state-copy bandwidth outside the step, rotating over n_caches
    caches (each bigger than the 256 MB last-level cache together) so that the
    bytes come from HBM.  Each cache holds P valid slots of arbitrary data."""
    import torch
    caches = [dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev) for _ in range(n_caches)]
    o = torch.empty((wl.B, wl.H, wl.Nq, wl.D), dtype=tdt, device=dev)
    lse = torch.empty((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
    src_o = torch.randn((wl.B, wl.H, wl.Nq, wl.D), device=dev).to(tdt)
    src_l = torch.randn((wl.B, wl.H, wl.Nq), device=dev) + 9.0
    for c in caches:
        for p in range(wl.P):
            c.store(p, src_o, src_l, step=0, stream=stream)
    torch.cuda.synchronize()
    merge_bytes = wl.merge_bytes()
    state_bytes = wl.state_bytes()

    def timed(fn, n):
        for i in range(n_caches):   # warm
            fn(i)
        b, e = dita.Event(), dita.Event()
        b.record(stream)
        for i in range(n):
            fn(i % n_caches)
        e.record(stream)
        return b.elapsed_ms(e) / n

    views = [([c.slot(p)[0] for p in range(wl.P)], [c.slot(p)[1] for p in range(wl.P)]) for c in caches]

    def merge(i):
        dita.dita_state_merge(views[i][0], views[i][1], o=o, lse=lse, stream=stream)

    def copy(i):   # slot 0 of cache i -> slot 1 of cache (i+1): one state read and one written
        src = caches[i].slot(0)
        caches[(i + 1) % n_caches].store(1, src[0], src[1], step=1, stream=stream)

    m_ms = min(timed(merge, 4 * n_caches) for _ in range(reps))
    c_ms = min(timed(copy, 4 * n_caches) for _ in range(reps))
    m_gbs = merge_bytes / (m_ms / 1e3) / 1e9
    c_gbs = 2 * state_bytes / (c_ms / 1e3) / 1e9
    log(f"[bench] isolated: merge {m_ms:.4f} ms = {m_gbs:.0f} GB/s; state copy {c_ms:.4f} ms = {c_gbs:.0f} GB/s")
    return {
        "merge": {"ms": m_ms, "bytes": merge_bytes, "GBps": m_gbs, "frac_hbm_peak": m_gbs / PEAK_HBM_GBS},
        "state_copy": {"ms": c_ms, "bytes": 2 * state_bytes, "GBps": c_gbs,
                       "frac_hbm_peak": c_gbs / PEAK_HBM_GBS},
        "note": f"rotating over {n_caches} caches of {wl.P} slots ({n_caches * caches[0].buffer.numel() / 1e9:.2f} GB)",
    }


def hbm_ceiling(dev, gib: int = 2, reps: int = 5):
    """An attainable HBM bandwidth on this GPU: torch's device-to-device copy of a
    `gib` GiB buffer (read + write), best of `reps`, beside the vendor's 8 TB/s."""
    import torch
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        dst.copy_(src)
        e.record()
        e.synchronize()
        ms = b.elapsed_time(e)
        best = ms if best is None else min(best, ms)
    gbs = 2 * n / (best / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"[bench] HBM ceiling: torch copy of {gib} GiB at {gbs:.0f} GB/s")
    # The merge's own mix, 16 reads to 1 write: torch's sum over the leading axis
    # of a [16, n] bf16 tensor (fp32 accumulation inside, bf16 out).
    rows, cols = 16, 24_192_000  # 16 slots of one 75,600-token state's O
    x = torch.ones(rows, cols, dtype=torch.bfloat16, device=dev)
    y = torch.empty(cols, dtype=torch.bfloat16, device=dev)
    torch.sum(x, dim=0, out=y)
    torch.cuda.synchronize()
    best_r = None
    for _ in range(reps):
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        torch.sum(x, dim=0, out=y)
        e.record()
        e.synchronize()
        ms = b.elapsed_time(e)
        best_r = ms if best_r is None else min(best_r, ms)
    r_gbs = (rows + 1) * cols * 2 / (best_r / 1e3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    log(f"[bench] torch 16-to-1 bf16 sum at {r_gbs:.0f} GB/s")
    return {"GBps": gbs, "frac_vendor_peak": gbs / PEAK_HBM_GBS,
            "how": f"torch device copy of {gib} GiB (read + write), best of {reps}",
            "sum16": {"GBps": r_gbs, "frac_vendor_peak": r_gbs / PEAK_HBM_GBS,
                      "how": f"torch.sum over dim 0 of a [16, {cols}] bf16 tensor "
                             f"(16 reads : 1 write, the merge's mix), best of {reps}"}}


def sustained_clock(run_step, seconds: float = 4.0):
    """The shader clock while rank-steps of the schedule run back to back: `amd-smi
    metric -c` (current clock of every XCD) polled from a thread, the first sample
    dropped; and the bf16 MFMA peak at that clock.  None when amd-smi is absent."""
    import re
    import shutil
    import subprocess
    import threading
    import torch
    exe = shutil.which("amd-smi")
    if not exe:
        return None
    samples = []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            try:
                out = subprocess.run([exe, "metric", "-c", "-g", "0"], capture_output=True, text=True,
                                     timeout=20).stdout
            except Exception:
                return
            clks = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", out)]
            if clks:
                samples.append(sum(clks) / len(clks))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            run_step(i)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    used = samples[1:] if len(samples) > 1 else samples
    if not used:
        return None
    mhz = float(np.median(used))   # median: a poll can land in a host-side gap between batches
    peak = PEAK_BF16_TFLOPS * mhz / 2400.0
    log(f"[bench] sustained shader clock {mhz:.0f} MHz over {len(used)} samples "
        f"(bf16 MFMA peak at that clock {peak:.0f} TFLOP/s)")
    return {"mhz_median": mhz, "mhz_mean": sum(used) / len(used), "mhz_min": min(used),
            "mhz_max": max(used), "samples": len(used),
            "steps_run": i, "peak_bf16_TFLOPs": peak,
            "how": "amd-smi metric -c (mean of the XCDs' current clocks) polled while the "
                   "schedule's rank-steps ran back to back; median of the polls; peak = "
                   "2.5 PFLOP/s x clock / 2.4 GHz"}


def attn_by_blocks(attn_ms, infos):
    """The attention launches of the timed steps grouped by their fresh-block count:
    launches, mean ms and TFLOP/s per group (the anchor steps' launches differ in
    shape from the others)."""
    groups = {}
    for ms, info in zip(attn_ms, infos):
        if info.n_fresh > 0:
            g = groups.setdefault(str(info.n_fresh), [0, 0.0, 0.0])
            g[0] += 1
            g[1] += ms
            g[2] += info.fresh_flops
    return {k: {"launches": n, "ms_mean": t / n, "TFLOPs": f / (t / 1e3) / 1e12}
            for k, (n, t, f) in sorted(groups.items(), key=lambda kv: int(kv[0]))}


def _call_times(dita, stream, call, reps: int):
    """GPU time of each of `reps` calls made back to back on `stream`: one call is
    queued ahead of the first event, so the host's launch work for each call
    overlaps the previous call and no interval includes GPU idle time waiting for
    the host.  Returns the per-call intervals (ms) between consecutive events."""
    evs = [dita.Event() for _ in range(reps + 1)]
    call(-1)
    evs[0].record(stream)
    for i in range(reps):
        call(i)
        evs[i + 1].record(stream)
    return [evs[i].elapsed_ms(evs[i + 1]) for i in range(reps)]  # waits for each later event


def lone_partial(dita, wl, tdt, dev, stream, q, kv0, reps: int = 20):
    """One dita_attn_partial call on one 75,600-token block (the rank's queries against
    one partition, all heads): after ~12 ms of warm-up calls, calls back to back on
    the launch stream, each on another block's K/V (read from HBM), HIP events
    between them, median of `reps`."""
    import torch
    ks, vs = kv0
    o = torch.empty((wl.B, wl.H, wl.Nq, wl.D), dtype=tdt, device=dev)
    lse = torch.empty((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
    for _ in range(30):  # ~12 ms of calls: the clock settles as under the step's load
        dita.dita_attn_partial(q, ks[1], vs[1], o=o, lse=lse, stream=stream)

    def call(i):
        j = 1 + (i + 1) % (wl.P - 1)
        dita.dita_attn_partial(q, ks[j], vs[j], o=o, lse=lse, stream=stream)

    times = _call_times(dita, stream, call, reps)
    ms = float(np.median(times))
    tf = wl.block_flops() / (ms / 1e3) / 1e12
    log(f"[bench] lone dita_attn_partial: {ms:.3f} ms = {tf:.0f} TFLOP/s")
    return {"ms_median": ms, "ms_min": float(np.min(times)), "flops": wl.block_flops(),
            "TFLOPs": tf, "frac": tf / PEAK_BF16_TFLOPS,
            "note": "one block, all heads: Q [1,40,4725,128] against one 4725-key partition; "
                    "calls back to back, each on another block's K/V"}


def short_query_partial(dita, wl, tdt, dev, stream, q, kv0, rows: int = 512, reps: int = 10):
    """One dita_attn_partial call with few query tiles: the first `rows` of the
    rank's queries against the whole sequence's keys (all partitions' K/V
    concatenated), all heads.  One 512-row tile per head leaves most compute
    units idle, so the library splits the tiles along the keys (reported with
    its launch layout).  Calls back to back, HIP events between them, median of
    `reps`."""
    import torch
    ks, vs = kv0
    rows = min(rows, wl.Nq)
    qs = q[:, :, :rows].contiguous()
    k = torch.cat([x for x in ks], dim=2)
    v = torch.cat([x for x in vs], dim=2)
    nk = k.shape[2]
    o = torch.empty_like(qs)
    lse = torch.empty((wl.B, wl.H, rows), dtype=torch.float32, device=dev)
    for _ in range(15):  # ~12 ms of calls, as for the lone call
        dita.dita_attn_partial(qs, k, v, o=o, lse=lse, stream=stream)
    times = _call_times(dita, stream,
                        lambda i: dita.dita_attn_partial(qs, k, v, o=o, lse=lse, stream=stream), reps)
    ms = float(np.median(times))
    flops = 4.0 * wl.B * wl.H * rows * nk * wl.D
    tf = flops / (ms / 1e3) / 1e12
    layout = dita.dita_attn_launch_info(wl.B, wl.H, rows, wl.D, 1, nk)
    log(f"[bench] short-query dita_attn_partial ({rows} x {nk}): {ms:.3f} ms = {tf:.0f} TFLOP/s, "
        f"{layout['split_units']} split units")
    del k, v
    return {"ms_median": ms, "flops": flops, "TFLOPs": tf, "frac": tf / PEAK_BF16_TFLOPS,
            "layout": layout,
            "note": f"Q [1,{wl.H},{rows},{wl.D}] against all {nk} keys: one query tile per head"}


def offload_overlap(dita, wl, tdt, dev, stream, q, kv, plan, reps: int = 3):
    """A non-anchor step whose composed far group was moved to pinned host memory:
    step time with the group resident, fetched on the step's stream, and fetched
    on a side stream while the fresh attention runs (no pre-merge)."""
    import torch
    cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev)
    o = torch.empty((wl.B, wl.H, wl.Nq, wl.D), dtype=tdt, device=dev)
    lse = torch.empty((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
    ks, vs = kv[0]
    dita.dita_attn_step(cache, q, ks, vs, np.zeros(wl.P, np.uint8), 0, o=o, lse=lse, stream=stream)
    mask = dita.dita_plan_mask(plan, 1, cache)
    cache.compose_runs(mask, stream=stream)
    groups = [p for p in cache.leaders() if cache.group(p)[1] > p]
    if not groups or wl.dtype != "bf16":
        return None
    side = torch.cuda.Stream(device=dev)
    ks1, vs1 = kv[1 % len(kv)]

    def one(offload, side_stream):
        if offload:
            for p in groups:
                cache.offload(p, stream=stream)
        torch.cuda.synchronize()
        b, e = dita.Event(), dita.Event()
        b.record(stream)
        _, _, info = dita.dita_attn_step(cache, q, ks1, vs1, mask, 1, o=o, lse=lse, stream=stream,
                                         side_stream=side_stream, min_premerge=64)
        e.record(stream)
        ms = b.elapsed_ms(e)
        assert info.fetched == (len(groups) if offload else 0)
        return ms

    res = {}
    for name, off, ss in (("resident", False, None), ("fetch_on_stream", True, None),
                          ("fetch_on_side_stream", True, side)):
        one(off, ss)
        res[name + "_ms"] = min(one(off, ss) for _ in range(reps))
    fetched_bytes = len(groups) * wl.state_bytes()
    res["fetched_bytes"] = fetched_bytes
    extra = res["fetch_on_stream_ms"] - res["resident_ms"]
    res["h2d_GBps_serial"] = fetched_bytes / (extra / 1e3) / 1e9 if extra > 0 else None
    res["hidden_fraction"] = ((res["fetch_on_stream_ms"] - res["fetch_on_side_stream_ms"]) / extra
                              if extra > 0 else None)
    res["note"] = (f"{len(groups)} composed group state(s) in pinned host memory, copied back by "
                   f"the step; fresh blocks {int((mask == 0).sum())}")
    log(f"[bench] offload: resident {res['resident_ms']:.3f} ms, fetch on stream "
        f"{res['fetch_on_stream_ms']:.3f} ms, on side stream {res['fetch_on_side_stream_ms']:.3f} ms")
    return res


def state_bytes_held(dita, cache, wl):
    """Bytes of the states a cache holds on the device (full: O and LSE; compact:
    codes, row scales and LSE), and what the same states would take in full."""
    rows = wl.B * wl.H * wl.Nq
    full_b, compact_b = rows * (2 * wl.D + 4), rows * (wl.D + 8)
    held = as_full = 0
    for p in range(wl.P):
        f = cache.format(p)
        if f in (dita.DITA_STATE_FULL, dita.DITA_STATE_COMPACT):
            held += compact_b if f == dita.DITA_STATE_COMPACT else full_b
            as_full += full_b
    return held, as_full


def trajectory(dita, wl, seed, dev, tdt, stream, compose_ahead=False, eplan=None, compact=False):
    """The schedule once from a cold cache beside an all-fresh reference (same library,
    same K/V, every partition recomputed): per-step error of the reused output, fresh
    blocks, step latency, and the contribution profile by partition distance."""
    import torch
    from workloads import Inputs
    inp = Inputs(wl, seed=seed)
    q = torch.from_numpy(inp.q).to(tdt).to(dev)
    if compact:
        cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev, slots=wl.P,
                                compact_slots=wl.P - 1)
    else:
        cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev)
    ref = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev)
    plan = dita.Plan(**wl.plan_fields())
    shape = (wl.B, wl.H, wl.Nq, wl.D)
    o = torch.empty(shape, dtype=tdt, device=dev)
    o_ref = torch.empty(shape, dtype=tdt, device=dev)
    lse = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    lse_ref = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    all_fresh = np.zeros(wl.P, dtype=np.uint8)
    out = {"fresh": [], "step_ms": [], "err_max_abs": [], "err_rel_fro": [], "lse_err_max_abs": []}
    contribution = None
    planner = None
    if eplan is not None:
        # error-guided planner: weights from the contribution kernel on all-fresh
        # steps, the local state's change measured after every step
        planner = dita.ErrorPlanner(wl.P, wl.q_part, eplan["group_size"], eplan["budget"],
                                    eplan["anchor_period"], eplan["fresh_weight"])
        prev_o = torch.zeros(shape, dtype=tdt, device=dev)
        prev_l = torch.zeros(shape[:3], dtype=torch.float32, device=dev)
        chg = torch.zeros(3, dtype=torch.float64, device=dev)
        out["planner"] = dict(eplan, est_err_reused=[], local_change=[])
    for s in range(wl.steps):
        k, v = inp.kv(s)
        ks, vs = upload_parts(k, wl, dev, tdt), upload_parts(v, wl, dev, tdt)
        del k, v
        if planner is None:
            mask = dita.dita_plan_mask(plan, s, cache)
        else:
            mask, est = planner.mask(s, cache=cache)
            out["planner"]["est_err_reused"].append(float(est[mask == 1].sum()))
        ev = (dita.Event(), dita.Event(), dita.Event())
        _, _, info = dita.dita_attn_step(cache, q, ks, vs, mask, s, o=o, lse=lse, stream=stream,
                                         events=(ev[0].handle, ev[1].handle, ev[2].handle))
        if planner is not None:
            if info.n_fresh == wl.P:
                planner.set_weights(list(cache.contrib(lse, stream=stream).cpu().numpy()))
            so, sl = cache.slot(wl.q_part)
            dita.dita_state_change(so, prev_o, sl, prev_l, roll=True, out=chg, stream=stream)
            if s > 0:
                d = float(chg[2].item())
                planner.observe(s, d)
                out["planner"]["local_change"].append(d)
            if eplan.get("compose_ahead") and s + 1 < wl.steps:
                # the planner's next mask is known once this step's change is observed
                cache.compose_runs(planner.mask(s + 1, cache=cache)[0], stream=stream)
        elif compose_ahead and s + 1 < wl.steps:
            cache.compose_runs(dita.dita_plan_mask(plan, s + 1, cache), stream=stream)
        if compact and s + 1 < wl.steps:
            nxt = dita.dita_plan_mask(plan, s + 1, cache)
            for p in range(wl.P):
                if nxt[p] == 1 and cache.format(p) == dita.DITA_STATE_FULL:
                    cache.compact(p, stream=stream)
            held, as_full = state_bytes_held(dita, cache, wl)
            out.setdefault("state_bytes_held", []).append(held)
            out.setdefault("state_bytes_if_full", []).append(as_full)
        dita.dita_attn_step(ref, q, ks, vs, all_fresh, s, o=o_ref, lse=lse_ref, stream=stream)
        torch.cuda.synchronize()
        d = o.float() - o_ref.float()
        out["fresh"].append(int(info.n_fresh))
        out["step_ms"].append(round(ev[0].elapsed_ms(ev[2]), 4))
        out["err_max_abs"].append(float(d.abs().max()))
        out["err_rel_fro"].append(float(torch.linalg.vector_norm(d) /
                                        torch.linalg.vector_norm(o_ref.float())))
        out["lse_err_max_abs"].append(float((lse - lse_ref).abs().max()))
        if s == 0:
            contribution = []
            for p in range(wl.P):
                _, lse_p = ref.slot(p)
                contribution.append(float(torch.exp(lse_p - lse_ref).mean()))
        log(f"[bench] trajectory step {s}: fresh {info.n_fresh}/{wl.P}  "
            f"err max-abs {out['err_max_abs'][-1]:.3e}  rel-Fro {out['err_rel_fro'][-1]:.3e}")
        del ks, vs
    run = 0.0
    out["err_running_max"] = []
    for e in out["err_max_abs"]:
        run = max(run, e)
        out["err_running_max"].append(run)
    out["fresh_blocks"] = sum(out["fresh"])
    out["fresh_fraction"] = out["fresh_blocks"] / (wl.steps * wl.P)
    out["contribution_by_distance"] = [
        {"distance": abs(p - wl.q_part), "partition": p, "mean_weight": contribution[p]}
        for p in range(wl.P)]
    out["reference"] = ("all-fresh step through the same library on the same K/V "
                        "(every partition recomputed = full attention)")
    if compact:
        held, full = sum(out["state_bytes_held"]), sum(out["state_bytes_if_full"])
        out["compact"] = {"state_bytes_saved_fraction": 1.0 - held / full if full else 0.0,
                          "note": "bytes held by cached states after each step's compaction, "
                                  "summed over the steps, against the same states held in full"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): sharding the "
              "rank-step across GPUs is not built.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    import partial_state_reuse_amd as dita
    import workloads
    from workloads import Inputs

    wl = workloads.get(args.workload)
    if args.fixed_radius >= 0:
        # a fixed distance schedule on the same shape and inputs (no anchors after step 0)
        wl = workloads.get(args.workload, policy=workloads.POLICY_DIST, radius=args.fixed_radius,
                           anchor_period=0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    n_sched = wl.steps
    n_res = n_sched if args.resident_steps <= 0 else min(args.resident_steps, n_sched)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} D={wl.D} N={wl.N} P={wl.P} Nk={wl.Nk} "
        f"dtype={wl.dtype}; generating {n_res} steps of inputs")
    t_gen = time.perf_counter()
    inp = Inputs(wl, seed=args.seed)
    q = torch.from_numpy(inp.q).to(tdt).to(dev)
    kv = []
    for s in range(n_res):
        k, v = inp.kv(s)
        kv.append((upload_parts(k, wl, dev, tdt), upload_parts(v, wl, dev, tdt)))
        log(f"[bench] inputs for schedule step {s} resident")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s")

    cache = dita.StateCache(wl.B, wl.H, wl.Nq, wl.D, tdt, wl.P, device=dev)
    plan = dita.Plan(**wl.plan_fields())
    o = torch.empty((wl.B, wl.H, wl.Nq, wl.D), dtype=tdt, device=dev)
    lse = torch.empty((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    side = torch.cuda.Stream(device=dev) if args.premerge else None

    def run(step_index, events=None):
        si = step_index % n_sched
        mask = dita.dita_plan_mask(plan, si, cache)
        ks, vs = kv[si % n_res]
        # The planner is deterministic: the step composes what the next step will
        # reuse (every partition is valid after a step, hence no cache for the mask).
        nxt = dita.dita_plan_mask(plan, (step_index + 1) % n_sched) if args.compose_ahead else None
        _, _, info = dita.dita_attn_step(cache, q, ks, vs, mask, step_index, o=o, lse=lse,
                                         stream=stream, events=events and events[:3],
                                         side_stream=side, compose_next=nxt)
        if events:
            assert dita.lib().dita_event_record(events[3], stream.cuda_stream) == 0
        return info

    # Device warm-up: whole cycles of the schedule, untimed, until args.device_warmup
    # seconds have passed (measured: after the host-side input generation the first
    # ~0.2 s of steps run 4-5% slower while the clock settles). The W warm-up steps
    # and the K timed steps follow, their step indices offset by whole cycles, so
    # they cover the same schedule positions as without it.
    under_profiler = any(k.startswith("ROCPROF") for k in os.environ) or \
        "rocprof" in os.environ.get("LD_PRELOAD", "")
    base = 0
    t0 = time.perf_counter()
    while args.device_warmup > 0 and time.perf_counter() - t0 < args.device_warmup:
        for s in range(n_sched):
            run(base + s)
        base += n_sched
        torch.cuda.synchronize()
    device_warmup = {"seconds": time.perf_counter() - t0, "steps": base,
                     "note": "whole schedule cycles run untimed before the --warmup steps"}
    if base:
        log(f"[bench] device warm-up: {base} steps in {device_warmup['seconds']:.2f} s")
    for s in range(args.warmup):
        run(base + s)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    K = args.steps
    evs = [(dita.Event(), dita.Event(), dita.Event(), dita.Event()) for _ in range(K)]
    t_begin, t_end = dita.Event(), dita.Event()
    infos = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for i in range(K):
        e = evs[i]
        infos.append(run(base + args.warmup + i, events=tuple(x.handle for x in e)))
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_begin.elapsed_ms(t_end)
    attn_ms = [e[0].elapsed_ms(e[1]) for e in evs]
    merge_ms = [e[1].elapsed_ms(e[2]) for e in evs]
    step_ms = [e[0].elapsed_ms(e[3]) for e in evs]
    compose_ms = [e[2].elapsed_ms(e[3]) for e in evs]
    fresh_flops = sum(i.fresh_flops for i in infos)
    fresh_blocks = sum(i.n_fresh for i in infos)
    merge_bytes = sum(i.merge_bytes for i in infos)
    launches = sum(1 for i in infos if i.n_fresh > 0)
    attn_s = sum(a for a, i in zip(attn_ms, infos) if i.n_fresh > 0) / 1e3
    achieved = fresh_flops / attn_s / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    merge_gbs = merge_bytes / (sum(merge_ms) / 1e3) / 1e9
    traffic_attn, traffic_merge = profiled_traffic(wl.name)
    if args.premerge or args.compose_ahead:
        traffic_merge = None   # the counters were taken on the P-way merge of the plain step
    log(f"[bench] timed {K} steps: {total_ms:.3f} ms (host wall {wall * 1e3:.1f} ms); "
        f"attention {sum(attn_ms):.3f} ms, merge {sum(merge_ms):.3f} ms")

    result = {
        "metric": "fresh-block attention TFLOP/s + ms per rank-step, 75,600-token DiT attn",
        "value": fresh_flops / (total_ms / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": wl.B, "H": wl.H, "D": wl.D, "tokens": wl.N,
            "grid_thw": list(wl.grid), "partitions": wl.P, "tokens_per_partition": wl.Nk,
            "query_partition": wl.q_part, "schedule_steps": n_sched, "resident_input_steps": n_res,
            "mask": {"policy": ["distance", "k-nearest", "random", "ramp"][wl.policy],
                     "radius": wl.radius, "radius_end": wl.radius_end, "k_nearest": wl.k_nearest,
                     "anchor_period": wl.anchor_period},
            "parallelism": "one rank's share on one GPU",
            "pipeline": {"premerge_side_stream": bool(args.premerge),
                         "compose_ahead": bool(args.compose_ahead)},
        },
        "fresh_blocks": fresh_blocks,
        "fresh_fraction": fresh_blocks / (K * wl.P),
        "fresh_tflop": fresh_flops / 1e12,
        "attn_ms_per_step": sum(attn_ms) / K,
        "merge_ms_per_step": sum(merge_ms) / K,
        "compose_ms_per_step": sum(compose_ms) / K,
        "premerge": bool(args.premerge),
        "compose_ahead": bool(args.compose_ahead),
        "merge_sources_per_step": [i.merge_sources for i in infos],
        "premerge_sources_per_step": [i.premerge_sources for i in infos],
        "step_ms": [round(x, 4) for x in step_ms],
        "step_ms_median": float(np.median(step_ms)),
        "step_ms_min": float(np.min(step_ms)),
        "device_warmup": device_warmup,
        "attn_by_fresh_blocks": attn_by_blocks(attn_ms, infos),
        "roofline": {
            "kernel": "attn_fwd_bf16_kernel (grouped fresh partial attention)"
            if wl.dtype == "bf16" else "attn_fwd_f32_kernel",
            "bound": "mfma" if wl.dtype == "bf16" else "alu",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic_attn,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, calibrated)",
            "launches": launches,
            "avg_launch_ms": attn_s * 1e3 / max(launches, 1),
            "flops_per_launch": fresh_flops / max(launches, 1),
        },
        "merge_in_step": {
            "kernel": "merge_kernel", "bound": None,
            "achieved": merge_gbs, "unit": "GB/s", "bytes_per_launch": merge_bytes / K,
            "traffic": traffic_merge,
            "avg_launch_ms": sum(merge_ms) / K,
            "note": ("algorithmic bytes / time of the step's final merge; it reads states the "
                     "attention launch has just written, which the 256 MB last-level cache "
                     "partly serves, so this is not an HBM figure (isolated.merge is)"),
        },
    }
    if wl.dtype == "bf16" and not args.no_clock and not under_profiler:
        clk = sustained_clock(lambda i: run(base + args.warmup + K + i))
        if clk:
            result["sustained_clock"] = clk
            result["roofline"]["peak_at_sustained_clock"] = clk["peak_bf16_TFLOPs"]
            result["roofline"]["frac_at_sustained_clock"] = achieved / clk["peak_bf16_TFLOPs"]
    result["isolated"] = isolated_bandwidth(dita, wl, tdt, dev, stream, q)
    result["hbm_ceiling"] = hbm_ceiling(dev)
    iso_m = result["isolated"]["merge"]
    iso_m["frac_measured_ceiling"] = iso_m["GBps"] / result["hbm_ceiling"]["GBps"]
    iso_m["frac_sum16"] = iso_m["GBps"] / result["hbm_ceiling"]["sum16"]["GBps"]
    if wl.dtype == "bf16":
        result["lone_attn_partial"] = lone_partial(dita, wl, tdt, dev, stream, q, kv[0])
        result["short_query_partial"] = short_query_partial(dita, wl, tdt, dev, stream, q, kv[0])
    if wl.steps > 1 and n_res > 1:
        result["offload"] = offload_overlap(dita, wl, tdt, dev, stream, q, kv, plan)
    if args.trajectory:
        del kv, cache
        torch.cuda.empty_cache()
        log("[bench] trajectory: the schedule from a cold cache beside an all-fresh reference")
        eplan = None
        if args.planner == "error":
            eplan = {"group_size": args.group_size, "budget": args.budget,
                     "anchor_period": args.planner_anchor, "fresh_weight": args.fresh_weight,
                     "compose_ahead": bool(args.planner_compose)}
        result["trajectory"] = trajectory(dita, wl, args.seed, dev, tdt, stream,
                                          compose_ahead=bool(args.compose_ahead), eplan=eplan,
                                          compact=bool(args.compact))
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
