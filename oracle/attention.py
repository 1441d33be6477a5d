"""fp64 dense-mask softmax attention (TEST INFRASTRUCTURE ONLY; see ``oracle``).

The method's attention is ordinary scaled dot-product softmax attention under
a block-causal mask: a query chunk sees its own tokens (both directions) and
the earlier chunks its context policy selects, never a later chunk.  Sources:
the Wave Forcing summary (aiany.app, mechanism paragraph) on chunk-wise causal
attention over earlier, cleaner chunks; Wan-Streamer v0.2 (Figure 1 and
"Model Formulation and Upgrade") on block-causal attention over one timeline.

This module writes that definition out literally: an additive mask of 0 / -inf
over every key the caller passes, S = scale * Q K^T + M, row softmax in fp64,
O = P V and LSE = log sum exp of the masked scores.  No blocking, no online
rescaling.

The pages fix no precision.  Inputs that the GPU consumes as bfloat16 are
rounded here with ``round_to_bf16`` (IEEE round-to-nearest-even on the upper
16 bits of binary32) and widened to fp64 before any arithmetic.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  NaN
    stays NaN (quietened), +-inf stays +-inf, finite values that round past
    the largest bfloat16 become +-inf, as IEEE rounding prescribes.
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lower = bits & 0xFFFF
    upper = bits >> 16
    halfway = 0x8000
    round_up = (lower > halfway) | ((lower == halfway) & ((upper & 1) == 1))
    upper = upper + round_up.astype(np.uint64)
    out = (upper << 16).astype(np.uint32)
    nan = np.isnan(a)
    out[nan] = (bits[nan].astype(np.uint32) | 0x00400000) & 0xFFFF0000
    return out.view(np.float32).reshape(a.shape)


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     mask: np.ndarray, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one head under an explicit additive mask.

    q: [Lq, d], k: [Lk, d], v: [Lk, dv], mask: [Lq, Lk] with entries 0 or -inf.
    Returns O [Lq, dv] and the natural-log LSE [Lq] of the masked scores.
    Every row must have at least one unmasked key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T) + mask
    rowmax = np.max(s, axis=1, keepdims=True)
    if not np.all(np.isfinite(rowmax)):
        raise ValueError("a query row has no unmasked key")
    e = np.exp(s - rowmax)
    z = np.sum(e, axis=1, keepdims=True)
    p = e / z
    o = p @ v
    lse = rowmax[:, 0] + np.log(z[:, 0])
    return o, lse


def softmax_rows(q, k, mask, scale):
    """The probability matrix P of ``masked_attention`` (used by the row-sum pin)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ k.T) + mask
    e = np.exp(s - np.max(s, axis=1, keepdims=True))
    return e / np.sum(e, axis=1, keepdims=True)


def slot_mask(key_slots: list, key_lens: list, ctx_def: list, lq: int) -> np.ndarray:
    """Dense [lq, sum(key_lens)] additive mask: 0 where the key's slot is in the
    node's context, -inf elsewhere.  The same for every query row of a chunk,
    since attention inside a chunk is bidirectional."""
    allowed = set(ctx_def)
    cols = []
    for s, n in zip(key_slots, key_lens):
        cols.append(np.full(n, 0.0 if s in allowed else -np.inf))
    row = np.concatenate(cols) if cols else np.zeros(0)
    return np.broadcast_to(row, (lq, row.shape[0]))
