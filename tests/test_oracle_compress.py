"""Pins of the compact state encoding (oracle/compress.py).

Exactly representable rows, ties, scaling by powers of two, the zero row and
the row maximum fix the encoding's values; a brute-force nearest-code search
in exact rational arithmetic fixes its rounding rule on many rows; the error
bound a/254 follows from the definition.  None of these re-types the
encoder's float32 formula."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.compress import CODE_MAX, bf16_round, compact_state, decode_rows, encode_rows
from oracle import StateCache, merge_states


def test_exactly_representable_row_and_ties():
    # a = 127: the scale is exactly 1 and each code is the value rounded half to even
    x = np.array([[127, -127, 0, 1, -1, 64, 2.5, 3.5, -2.5, -3.5, 126.5, 0.5, 1.5]], np.float32)
    codes, scale = encode_rows(x)
    assert scale.tolist() == [1.0]
    assert codes.tolist() == [[127, -127, 0, 1, -1, 64, 2, 4, -2, -4, 126, 0, 2]]
    assert np.array_equal(decode_rows(codes, scale), np.rint(x).astype(np.float64))


@pytest.mark.parametrize("k", [-20, -7, 0, 3, 40])
def test_power_of_two_scaling(k):
    rng = np.random.default_rng(k + 100)
    x = bf16_round(rng.standard_normal((16, 64)))
    c0, s0 = encode_rows(x)
    c1, s1 = encode_rows(x * np.float32(2.0 ** k))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** k))


def test_zero_row_and_row_maximum():
    rng = np.random.default_rng(1)
    x = bf16_round(rng.standard_normal((50, 128)))
    x[7] = 0.0
    codes, scale = encode_rows(x)
    assert scale[7] == 0.0 and not codes[7].any()
    assert np.array_equal(decode_rows(codes, scale)[7], np.zeros(128))
    rows = np.arange(50) != 7
    imax = np.argmax(np.abs(x), axis=-1)
    top = codes[np.arange(50), imax]
    assert np.array_equal(np.abs(top[rows]), np.full(49, CODE_MAX))
    assert np.array_equal(np.sign(top[rows]), np.sign(x[np.arange(50), imax][rows]).astype(np.int8))
    assert np.all(np.abs(codes.astype(np.int32)) <= CODE_MAX)


def _nearest_code_exact(row):
    """Brute force: the integer k in [-127, 127] nearest to x * 127 / a in exact
    rational arithmetic, ties to the even k."""
    a = max(abs(Fraction(float(v))) for v in row)
    out = []
    for v in row:
        if a == 0:
            out.append(0)
            continue
        t = Fraction(float(v)) * CODE_MAX / a
        best = min(range(-CODE_MAX, CODE_MAX + 1), key=lambda k: (abs(t - k), k % 2))
        out.append(best)
    return out


def test_rounding_rule_by_brute_force():
    rng = np.random.default_rng(2)
    rows = [bf16_round(rng.standard_normal(12) * rng.choice([1e-3, 1.0, 50.0])) for _ in range(300)]
    # constructed halves: a = 127 * 2^e, values (n + 1/2) * 2^e
    for e in (-4, 0, 5):
        n = rng.integers(-126, 126, 12).astype(np.float64)
        r = ((n + 0.5) * 2.0 ** e).astype(np.float32)
        r[0] = np.float32(127 * 2.0 ** e)
        rows.append(bf16_round(r))
    for r in rows:
        codes, _ = encode_rows(r[None])
        assert codes[0].tolist() == _nearest_code_exact(r)


def test_error_bound_of_the_definition():
    rng = np.random.default_rng(3)
    x = bf16_round(rng.standard_normal((400, 128)) * rng.uniform(0.01, 3.0, (400, 1)))
    codes, scale = encode_rows(x)
    a = np.max(np.abs(x.astype(np.float64)), axis=-1, keepdims=True)
    err = np.abs(decode_rows(codes, scale) - x.astype(np.float64))
    assert np.all(err <= a / 254 + a * 2.0 ** -21)
    assert np.max(err / (a / 254)) > 0.9        # the bound is reached, not loose by a factor


def test_rejects_values_that_are_not_bf16():
    with pytest.raises(ValueError):
        encode_rows(np.array([[1.0 + 2.0 ** -12]], np.float32))


def test_compacted_state_in_a_merge():
    """A merge over compacted states equals the merge over the decoded values and
    stays within the per-row code step of the merge over the full states."""
    rng = np.random.default_rng(4)
    P, shape = 4, (1, 2, 30, 64)
    states = [(rng.standard_normal(shape) * 0.5, rng.standard_normal(shape[:3]) + 5.0) for _ in range(P)]
    cache = StateCache(P)
    for p, st in enumerate(states):
        cache.store(p, st, 0)
        cache.compact(p)
    o_c, l_c = merge_states([cache.slots[p] for p in range(P)])
    o_f, l_f = merge_states(states)
    assert np.array_equal(l_c, l_f)                  # LSE is kept exactly
    lses = np.stack([s[1] for s in states])
    w = np.exp(lses - l_f[None])
    steps = []
    for o, _ in states:
        x = bf16_round(o)
        steps.append(np.max(np.abs(x.astype(np.float64)), axis=-1) / 127)
    bound = np.sum(w * np.stack(steps), axis=0)[..., None] * 0.5 + 2.0 ** -8
    assert np.all(np.abs(o_c - o_f) <= bound)
    d = [compact_state(s) for s in states]
    o_d, _ = merge_states(d)
    assert np.max(np.abs(o_d - o_c)) == 0.0
