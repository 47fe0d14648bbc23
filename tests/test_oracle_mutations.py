"""Planted mistakes in the oracle are caught by its pins.

Each case copies the oracle package into a temporary directory, plants one
plausible mistake in it by a textual edit (a dropped term, a wrong sign,
index, axis or operand, a changed constant or comparison), imports the copy
as ``oracle`` and runs the pin tests against it on the CPU.  At least one pin
must fail for every planted mistake; the unmodified copy must pass them all.

The pins are the oracle tests (closed forms, library reductions, brute force,
invariants, the published SplitMix64 value, closed-form mask counts) and, for
the Bernoulli planner's stream seeding, which the pages leave open, the
bit-exact agreement with the library's independent C++ planner.
"""

from __future__ import annotations

import importlib.util
import inspect
import itertools
import pathlib
import shutil
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
PINS = {
    "attention.py": ["test_oracle_attention", "test_oracle_merge"],
    "cache.py": ["test_oracle_merge", "test_oracle_groups", "test_oracle_compress"],
    "compress.py": ["test_oracle_compress"],
    "planner.py": ["test_oracle_planner", "test_abi"],
    "error_planner.py": ["test_oracle_error_planner", "test_abi"],
}

# (file, what the mistake is, text in the oracle, replacement)
MUTATIONS = [
    ("compress.py", "scale a/128", "a / np.float32(CODE_MAX)", "a / np.float32(128)"),
    ("compress.py", "codes truncated instead of rounded", "q = np.rint(t / safe[..., None])",
     "q = np.trunc(t / safe[..., None])"),
    ("compress.py", "ties rounded away from zero", "q = np.rint(t / safe[..., None])",
     "q = np.trunc(t / safe[..., None] + np.copysign(np.float32(0.5), t))"),
    ("compress.py", "row maximum without the magnitude", "a = np.max(np.abs(x), axis=-1)",
     "a = np.max(x, axis=-1)"),
    ("compress.py", "codes scaled to 126", "t = x * np.float32(CODE_MAX)",
     "t = x * np.float32(CODE_MAX - 1)"),
    ("compress.py", "decode divides by the scale", "(c * s[..., None])", "(c / np.where(s > 0, s, 1)[..., None])"),
    ("compress.py", "encoding the unrounded state",
     "encode_rows(bf16_round(np.asarray(o, dtype=np.float64)))",
     "encode_rows(np.asarray(o, dtype=np.float64).astype(np.float32))"),
    ("cache.py", "compaction not kept", "self.slots[p] = compact_state(self.slots[p])",
     "compact_state(self.slots[p])"),
    ("attention.py", "default scale 1/D", "1.0 / math.sqrt(head_dim)", "1.0 / head_dim"),
    ("attention.py", "scores against V instead of K",
     "s = scale * np.matmul(q, np.swapaxes(k, -1, -2))",
     "s = scale * np.matmul(q, np.swapaxes(v, -1, -2))"),
    ("attention.py", "score sign", "s = scale * np.matmul", "s = -scale * np.matmul"),
    ("attention.py", "row max over the query axis",
     "m = np.max(s, axis=-1, keepdims=True)", "m = np.max(s, axis=-2, keepdims=True)"),
    ("attention.py", "LSE without the max term",
     "lse = m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True))",
     "lse = np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True))"),
    ("attention.py", "denominator summed over the query axis",
     "np.sum(np.exp(s - m), axis=-1, keepdims=True)",
     "np.sum(np.exp(s - m), axis=-2, keepdims=True)"),
    ("attention.py", "output not normalised",
     "o = np.matmul(np.exp(s - lse), v)", "o = np.matmul(np.exp(s - m), v)"),
    ("attention.py", "output from K instead of V",
     "o = np.matmul(np.exp(s - lse), v)", "o = np.matmul(np.exp(s - lse), k)"),
    ("attention.py", "merge weights with the wrong sign",
     "np.exp(lses - m_safe[None])", "np.exp(m_safe[None] - lses)"),
    ("attention.py", "merged LSE without the max term",
     "m_safe + np.log(np.where(empty, 1.0, total))", "np.log(np.where(empty, 1.0, total))"),
    ("attention.py", "merged output not normalised",
     "o = np.sum((w / denom[None])[..., None] * outs, axis=0)",
     "o = np.sum(w[..., None] * outs, axis=0)"),
    ("attention.py", "all-neutral rows merge to LSE 0",
     "lse = np.where(empty, -np.inf,", "lse = np.where(empty, 0.0,"),
    ("cache.py", "reuse mask read inverted", "        if not reuse[p]:\n            cache.store(",
     "        if reuse[p]:\n            cache.store("),
    ("cache.py", "fresh state from the wrong V partition",
     "partial_state(q, k_parts[p], v_parts[p], scale)",
     "partial_state(q, k_parts[p], v_parts[0], scale)"),
    ("cache.py", "stamp not recorded", "self.stamp[p] = step", "self.stamp[p] = 0"),
    ("cache.py", "merge over the fresh slots only",
     "o, lse = merge_states([cache.slots[p] for p in cache.leaders()])",
     "o, lse = merge_states([cache.slots[p] for p in cache.leaders() if not reuse[p]] or [cache.slots[0]])"),
    ("cache.py", "group composed from its first state only",
     "state = merge_states([self.slots[p] for p in heads])",
     "state = merge_states([self.slots[p] for p in heads[:1]])"),
    ("cache.py", "group stamp from the newest member",
     "oldest = min(int(self.stamp[p]) for p in heads)", "oldest = max(int(self.stamp[p]) for p in heads)"),
    ("cache.py", "group reused when any member is reused",
     "if last > first and not reuse[first:last + 1].all():",
     "if last > first and not reuse[first:last + 1].any():"),
    ("cache.py", "group range one short", "while last + 1 < self.P and self.group[last + 1] == first:",
     "while last + 2 < self.P and self.group[last + 1] == first:"),
    ("cache.py", "reuse of an empty slot not rejected",
     "        if reuse[p] and not cache.valid[p]:\n            raise RuntimeError(f\"partition {p} is marked reuse but its slot is empty\")\n    reuse = effective_reuse",
     "        if False:\n            raise RuntimeError(f\"partition {p} is marked reuse but its slot is empty\")\n    reuse = effective_reuse"),
    ("cache.py", "compose-ahead run ends one short",
     "        while p + 1 < cache.P and reuse[p + 1]:\n",
     "        while p + 2 < cache.P and reuse[p + 1]:\n"),
    ("cache.py", "compose-ahead keeps groups reaching outside the run",
     "if cache.group_range(i)[0] >= a and cache.group_range(i)[1] <= b]",
     "if cache.group_range(i)[0] >= a]"),
    ("error_planner.py", "contribution without the merged LSE",
     "w[ok] = np.exp(lp[ok] - lse[ok])", "w[ok] = np.exp(lp[ok])"),
    ("error_planner.py", "contribution averaged over partitions, not rows",
     "out[p] = float(np.sum(w)) / lse.size", "out[p] = float(np.sum(w)) / len(lse_parts)"),
    ("error_planner.py", "state change not relative", "return num / den", "return num"),
    ("error_planner.py", "growth counted from the stamp step itself",
     "for t in range(int(stamp[p]) + 1, step + 1):", "for t in range(int(stamp[p]), step + 1):"),
    ("error_planner.py", "prediction peeks at the planned step",
     "seen = sorted(u for u in self.delta if u <= step - 1)",
     "seen = sorted(u for u in self.delta if u <= step)"),
    ("error_planner.py", "local partition inside its group's decision",
     "members = [p for p in range(a, b + 1) if p != q]", "members = [p for p in range(a, b + 1)]"),
    ("error_planner.py", "groups taken in decreasing error",
     "candidates.sort(key=lambda c: (c[0], c[1]))", "candidates.sort(key=lambda c: (-c[0], c[1]))"),
    ("error_planner.py", "high-contribution threshold exclusive",
     "any(self.weights[p] >= self.fresh_weight for p in members)",
     "any(self.weights[p] > self.fresh_weight for p in members)"),
    ("error_planner.py", "error without the weight", "err[p] = self.weights[p] * growth",
     "err[p] = growth"),
    ("planner.py", "SplitMix64 multiplier typo", "0xBF58476D1CE4E5B9", "0xBF58476D1CE4E5B8"),
    ("planner.py", "SplitMix64 shift", "z = ((z ^ (z >> 30))", "z = ((z ^ (z >> 31))"),
    ("planner.py", "SplitMix64 output before the gamma step",
     "self.state = (self.state + self.GAMMA) & _MASK64\n        z = self.state",
     "z = self.state\n        self.state = (self.state + self.GAMMA) & _MASK64"),
    ("planner.py", "distance radius exclusive",
     "reuse[p] = 1 if abs(p - q) > r else 0", "reuse[p] = 1 if abs(p - q) >= r else 0"),
    ("planner.py", "k-nearest ties to the higher index",
     "key=lambda p: (abs(p - q), p)", "key=lambda p: (abs(p - q), -p)"),
    ("planner.py", "Bernoulli bit from the low end", "reuse[p] = draw >> 63", "reuse[p] = draw & 1"),
    ("planner.py", "Bernoulli stream seeded without the seed shift",
     "SplitMix64(((plan.seed << 32) ^ step) & _MASK64)", "SplitMix64((plan.seed ^ step) & _MASK64)"),
    ("planner.py", "ramp radius floored", "return (2 * n + d) // (2 * d)", "return n // d"),
    ("planner.py", "local partition not forced fresh", "    reuse[q] = 0\n", "\n"),
    ("planner.py", "anchor off by one",
     "step % plan.anchor_period == 0", "(step + 1) % plan.anchor_period == 0"),
    ("planner.py", "cold slots not forced fresh", "reuse[valid == 0] = 0", "pass"),
]


def _param_sets(fn):
    """Argument sets of a test function from its parametrize marks (none: one empty set)."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [{}]
    axes = []
    for m in marks:
        names, values = m.args[0], m.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        axis = []
        for v in values:
            v = v.values if hasattr(v, "values") and not isinstance(v, (tuple, list)) else v
            v = tuple(v) if len(names) > 1 else (v,)
            axis.append(dict(zip(names, v)))
        axes.append(axis)
    return [dict(itertools.chain.from_iterable(d.items() for d in combo))
            for combo in itertools.product(*axes)]


def _run_pins(pkg_parent: pathlib.Path, modules):
    """Run the pin tests of ``modules`` with ``oracle`` imported from ``pkg_parent``;
    return the ids of the tests that failed and the number of cases run."""
    saved = {k: v for k, v in sys.modules.items() if k == "oracle" or k.startswith("oracle.")}
    for k in saved:
        del sys.modules[k]
    sys.path.insert(0, str(pkg_parent))
    failed, n_run = [], 0
    try:
        for name in modules:
            spec = importlib.util.spec_from_file_location(f"_pin_{name}", ROOT / "tests" / f"{name}.py")
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            for tname, fn in inspect.getmembers(mod, inspect.isfunction):
                if not tname.startswith("test_") or fn.__module__ != mod.__name__:
                    continue
                params = set(inspect.signature(fn).parameters)
                for kwargs in _param_sets(fn):
                    if set(kwargs) != params:
                        break   # needs a fixture: not a pin of the oracle
                    n_run += 1
                    try:
                        fn(**kwargs)
                    except Exception as exc:   # an assertion, or the mutant crashed
                        failed.append(f"{name}::{tname}[{kwargs}]: {type(exc).__name__}")
                        break
    finally:
        sys.path.remove(str(pkg_parent))
        for k in [k for k in sys.modules if k == "oracle" or k.startswith("oracle.")]:
            del sys.modules[k]
        sys.modules.update(saved)
    return failed, n_run


def _copy_oracle(tmp_path: pathlib.Path) -> pathlib.Path:
    dst = tmp_path / "oracle"
    shutil.copytree(ROOT / "oracle", dst, ignore=shutil.ignore_patterns("__pycache__"))
    return dst


def test_unmodified_copy_passes_every_pin(tmp_path):
    _copy_oracle(tmp_path)
    modules = sorted({m for ms in PINS.values() for m in ms})
    failed, n_run = _run_pins(tmp_path, modules)
    assert failed == []
    print(f"{n_run} pin cases")
    assert n_run >= 70, n_run   # every parametrised pin case ran


@pytest.mark.parametrize("fname,what,old,new", MUTATIONS, ids=[m[1] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, fname, what, old, new):
    pkg = _copy_oracle(tmp_path)
    path = pkg / fname
    src = path.read_text()
    assert src.count(old) == 1, f"the text to mutate must occur once in {fname}: {old!r}"
    path.write_text(src.replace(old, new))
    failed, _ = _run_pins(tmp_path, PINS[fname])
    assert failed, f"no pin caught: {what}"
