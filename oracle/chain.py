"""Toy denoiser chain around the attention (TEST INFRASTRUCTURE ONLY; see ``oracle``).

The pages carry no model weights, so the steps on either side of the
attention (the QKV projection before it, the sampler between denoising
levels) are a seeded stand-in.  This module writes its definition out once,
serially and in fp64:

* D = heads * head_dim.  Each layer l has a projection W_l [3D][D]; row o
  holds the weights of output column o (a seeded input, bf16 values).
* The input A of a node at layer 0 is, for the first update U(i,K) of a
  chunk, the chunk's seeded noise; for every later node of the chunk (U(i,j)
  with j < K, and the refresh R(i)) it is the last-layer attention output of
  the chunk's previous node.  This is the data flow the Wave Forcing summary
  (mechanism paragraph) and the design-space paper (Figure 2) describe: a
  chunk's next denoising step consumes its current one's result, and the
  refresh pass consumes the fully denoised chunk.
* At layer l:  [Q | K | V] = bf16( (A W_l^T) / rms(A) ),  with
  rms(a) = sqrt(mean_c a_c^2 + 1e-6) per token.  Q is the node's query; K and
  V are written to the node's own slot (chunk, level) of layer l's cache.
  O = block-causal attention over the node's context (``oracle.attention``)
  and the next layer's A = bf16(O).
* The node's result is the last layer's bf16(O).

Rounding points (bf16 of the projection and of O) are part of the
definition; values are computed in fp64 and rounded through binary32.
Every node is run in the serial schedule's order, with each node's context
recomputed from phi (``oracle.plan.context``), so routing errors of a plan
cannot leak in.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention, round_to_bf16, slot_mask
from .plan import Params, context

RMS_EPS = 1e-6


def bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to bfloat16 (through binary32), returned as fp64."""
    return round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def project(a: np.ndarray, w: np.ndarray, heads: int, head_dim: int):
    """(Q, K, V), each [L, heads, head_dim]: bf16((a w^T) / rms(a)).

    a: [L, D] fp64 (bf16 values); w: [3D, D] fp64 (bf16 values)."""
    d_model = heads * head_dim
    a = np.asarray(a, np.float64)
    y = a @ np.asarray(w, np.float64).T
    inv = 1.0 / np.sqrt(np.mean(a * a, axis=1) + RMS_EPS)
    y = bf16(y * inv[:, None])
    L = a.shape[0]
    q = y[:, :d_model].reshape(L, heads, head_dim)
    k = y[:, d_model:2 * d_model].reshape(L, heads, head_dim)
    v = y[:, 2 * d_model:].reshape(L, heads, head_dim)
    return q, k, v


def chain_rollout(p: Params, plan: dict, layers: int, heads: int, head_dim: int, noise, weight,
                  scale: float):
    """Run the toy chain over `plan` (any schedule; executed round by round).

    noise(chunk) -> [L, D] bf16 values; weight(layer) -> [3D, D] bf16 values.
    Returns {(chunk, level): (result [L, D], [O_0 .. O_{layers-1}] each [L, heads, head_dim])}.
    Requires no conditioning slots and query rows = chunk tokens.
    """
    if p.cond_len != 0 or (p.query_len not in (0, p.chunk_len)):
        raise ValueError("the toy chain needs cond_len = 0 and query_len = chunk_len")
    caches = [dict() for _ in range(layers)]
    state: dict[int, np.ndarray] = {}
    nodes = plan["nodes"]
    rnb = plan["round_node_begin"]
    out = {}
    for t in range(plan["num_rounds"]):
        rnodes = nodes[rnb[t]:rnb[t + 1]]
        # K/V of every node of the round first (same-round reads of lower chunks),
        # layer by layer: a node's layer-l K/V depend on its layer l-1 output.
        a_cur = {}
        for (c, lv, *_r) in rnodes:
            a_cur[(c, lv)] = np.asarray(state[c] if c in state else noise(c), np.float64)
        outs_l = {(c, lv): [] for (c, lv, *_r) in rnodes}
        for layer in range(layers):
            w = weight(layer)
            qs = {}
            for (c, lv, *_r) in rnodes:
                q, k, v = project(a_cur[(c, lv)], w, heads, head_dim)
                caches[layer][(c, lv)] = (k, v)
                qs[(c, lv)] = q
            for (c, lv, *_r) in rnodes:
                ctx = context(p, c, lv)
                cache = caches[layer]
                for s in ctx:
                    if s not in cache:
                        raise RuntimeError(f"node ({c},{lv}) in round {t} reads unwritten slot {s}")
                keys = list(cache.keys())
                lens = [cache[s][0].shape[0] for s in keys]
                kall = np.concatenate([cache[s][0] for s in keys], axis=0)
                vall = np.concatenate([cache[s][1] for s in keys], axis=0)
                q = qs[(c, lv)]
                mask = slot_mask(keys, lens, ctx, q.shape[0])
                o = np.zeros((q.shape[0], heads, head_dim))
                for h in range(heads):
                    o[:, h, :], _ = masked_attention(q[:, h, :], kall[:, h, :], vall[:, h, :], mask, scale)
                o = bf16(o)
                outs_l[(c, lv)].append(o)
                a_cur[(c, lv)] = o.reshape(q.shape[0], heads * head_dim)
        for (c, lv, *_r) in rnodes:
            state[c] = a_cur[(c, lv)]
            out[(c, lv)] = (a_cur[(c, lv)], outs_l[(c, lv)])
    return out
