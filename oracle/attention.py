"""Attention states in float64: partial state, LSE merge, full attention.

Test infrastructure only (see the package docstring).

An *attention state* of a query block against one K/V context partition is
the pair (output, log-sum-exp), the composable object of the DiTango page,
Methodology > 2. State-Centric Parallel Runtime > "State Composition".

Readings taken where the page is silent:

* the output of a partial state is normalised by that partition's own
  softmax denominator, so every output row is a convex combination of the
  partition's value rows; the raw, unnormalised form is exp(LSE) * O;
* the softmax scale defaults to 1/sqrt(D) and is a parameter;
* attention is bidirectional: no mask inside a partition (the page's problem
  statement says DiTs attend over the whole spatiotemporal sequence);
* LSE uses the natural logarithm.

Arrays are [..., N, D] (leading dims are batch and heads); LSE is [..., Nq].
All arithmetic is float64; inputs are widened exactly with ``astype``.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

State = Tuple[np.ndarray, np.ndarray]


def softmax_scale(head_dim: int) -> float:
    """Default softmax temperature 1/sqrt(D) (scaled dot-product attention)."""
    return 1.0 / math.sqrt(head_dim)


def _f64(x) -> np.ndarray:
    return np.asarray(x).astype(np.float64, copy=False)


def partial_state(q, k, v, scale: float | None = None) -> State:
    """State of queries ``q`` against one context partition (``k``, ``v``).

    Written out from its definition:

        S     = scale * Q K^T
        m     = rowmax(S)
        LSE   = m + ln( sum_j exp(S_ij - m) )
        O     = exp(S - LSE) V

    Returns (O [..., Nq, D], LSE [..., Nq]) in float64.  A partition with no
    keys has the neutral state (0, -inf).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if scale is None:
        scale = softmax_scale(q.shape[-1])
    nq, nk = q.shape[-2], k.shape[-2]
    if nk == 0:
        lead = np.broadcast_shapes(q.shape[:-2], k.shape[:-2])
        return (np.zeros(lead + (nq, v.shape[-1])), np.full(lead + (nq,), -np.inf))
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    m = np.max(s, axis=-1, keepdims=True)
    lse = m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True))
    o = np.matmul(np.exp(s - lse), v)
    return o, lse[..., 0]


def merge_states(states: Iterable[State]) -> State:
    """Compose attention states exactly by their log-sum-exp weights.

    For states (O_p, LSE_p), p = 1..P, row by row:

        M   = max_p LSE_p            (over finite LSE_p)
        w_p = exp(LSE_p - M)
        L   = sum_p w_p
        LSE = M + ln L
        O   = sum_p (w_p / L) O_p

    A state with LSE = -inf has weight 0 (the neutral element).  A row where
    every LSE_p is -inf merges to (0, -inf).
    """
    states = [(_f64(o), _f64(l)) for o, l in states]
    if not states:
        raise ValueError("merge_states needs at least one state")
    lses = np.stack([l for _, l in states], axis=0)          # [P, ..., Nq]
    outs = np.stack([o for o, _ in states], axis=0)          # [P, ..., Nq, D]
    m = np.max(lses, axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - m_safe[None]))
    total = np.sum(w, axis=0)
    denom = np.where(empty, 1.0, total)
    o = np.sum((w / denom[None])[..., None] * outs, axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    return o, lse


def full_attention(q, k_parts: Sequence, v_parts: Sequence, scale: float | None = None) -> State:
    """Attention of ``q`` over the concatenation of all K/V partitions.

    This is the result that merging all-fresh partial states must reproduce:
    sum_p exp(LSE_p) equals the full softmax denominator, and re-weighting
    each O_p by exp(LSE_p - LSE) restores the global softmax weights.
    """
    k = np.concatenate([_f64(x) for x in k_parts], axis=-2)
    v = np.concatenate([_f64(x) for x in v_parts], axis=-2)
    return partial_state(q, k, v, scale)
