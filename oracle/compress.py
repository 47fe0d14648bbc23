"""Compact encoding of a cached attention state -- TEST INFRASTRUCTURE ONLY.

The DiTango page names the memory held by cached states as a limitation of
the method and cache compression as future work (section "Significance and
Claims", closing paragraph on limitations).  The page gives no format; the
reading taken here (plainest one that halves the bytes of a bf16 state while
keeping every element within a fixed fraction of its row's magnitude):

* a state's output O is stored as bf16 by the library; compaction encodes
  those stored values row by row (a row = one query of one head);
* per row: a = max_d |O_d|; scale s = a / 127; code_d = round-half-even of
  O_d * 127 / a, an integer in [-127, 127] kept as int8; a row of zeros has
  s = 0 and all codes 0;
* the state's LSE is kept exactly (float32);
* the value a merge uses is code_d * s.

All steps are float32 operations with one rounding each, so the encoding is
reproducible bit for bit: O_d * 127 is exact for bf16 values (8 + 7
significant bits), the quotient and the scale are correctly rounded
divisions, and the decoded value is one correctly rounded product.  Every
element then lies within s/2 = a/254 of its stored value (plus the two
roundings of the scale and the product).

Bytes per row at head dimension D: D codes + 4 (scale) + 4 (LSE), against
2D + 4 for the bf16 state: 136 against 260 at D = 128.
"""

from __future__ import annotations

import numpy as np

CODE_MAX = 127


def bf16_round(x) -> np.ndarray:
    """Values rounded to the nearest bfloat16 (ties to even), returned as float32.
    Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def encode_rows(o) -> tuple:
    """Encode bf16-representable values ``o`` [..., D] (given as float32 or wider,
    each exactly a bfloat16) row by row.  Returns (codes int8 [..., D], scale
    float32 [...])."""
    x = np.asarray(o, dtype=np.float32)
    if not np.array_equal(bf16_round(x), x):
        raise ValueError("compaction encodes bf16 values")
    a = np.max(np.abs(x), axis=-1)
    t = x * np.float32(CODE_MAX)                      # exact for bf16 values
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    q = np.rint(t / safe[..., None])                  # float32 quotient, rounded once
    q = np.where(a[..., None] > 0, q, np.float32(0.0))
    scale = np.where(a > 0, a / np.float32(CODE_MAX), np.float32(0.0)).astype(np.float32)
    return q.astype(np.int8), scale


def decode_rows(codes, scale) -> np.ndarray:
    """The values a merge uses: code * scale, one float32 product, as float64."""
    c = np.asarray(codes).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32)
    return (c * s[..., None]).astype(np.float64)


def compact_state(state):
    """A cached state (O, LSE) as the cache holds it after compaction: O narrowed
    to bf16 (what the library stores), encoded and decoded; LSE unchanged."""
    o, lse = state
    codes, scale = encode_rows(bf16_round(np.asarray(o, dtype=np.float64)))
    return decode_rows(codes, scale), np.asarray(lse, dtype=np.float64)
