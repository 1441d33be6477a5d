"""Serial rollout of a plan against a dict cache (TEST INFRASTRUCTURE ONLY).

Executes the rounds of a plan in order.  For each round: every write of the
round stores fresh K/V in a dict keyed by logical slot (chunk, level); then
every node attends, with a dense mask built over all slots currently in the
dict.  The mask comes from the node's context recomputed from phi
(``oracle.plan.context``), not from the plan's context lists, so a wrong
gather list in a plan shows up as an output mismatch.  A context slot missing
from the dict is a hard error (an early read).

A slot is dropped from the dict once no later node's recomputed context
mentions it; this only bounds memory, the mask already gives such slots -inf.

Inputs are supplied by callables so that the oracle never generates data:
``get_kv(chunk, level)`` returns (K, V) as [len, heads, d] arrays and
``get_q(chunk, level)`` returns Q as [Lq, heads, d].  Both return the exact
values the GPU consumes (already bf16-representable), widened here to fp64.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention, slot_mask
from .plan import Params, context


def rollout(p: Params, plan: dict, get_q, get_kv, scale: float, rows=None,
            heads=None, want=None):
    """Run `plan` serially; return {(chunk, level): (O [rows, h, dv], LSE [h, rows])}.

    rows(chunk, level) -> index array of query rows to compute (default: all).
    heads: iterable of head indices (default: all).
    want: set of (chunk, level) nodes to compute (default: all); the rollout
    stops once they are done.
    """
    cache: dict[tuple[int, int], tuple[np.ndarray, np.ndarray]] = {}
    nodes = plan["nodes"]
    rnb = plan["round_node_begin"]
    writes = plan["writes"]
    # Recompute every node's context from phi for the liveness bound.
    future_reads: dict[tuple[int, int], int] = {}
    for (c, lv, *_rest) in nodes:
        for s in context(p, c, lv):
            future_reads[s] = future_reads.get(s, 0) + 1
    out = {}
    for t in range(plan["num_rounds"]):
        rnodes = nodes[rnb[t]:rnb[t + 1]]
        for (c, lv, kind, rnd, qo, ql, cb, cc, wb, wc) in rnodes:
            for (wc_, wl, _pid, _len) in writes[wb:wb + wc]:
                k, v = get_kv(wc_, wl)
                cache[(wc_, wl)] = (np.asarray(k, np.float64), np.asarray(v, np.float64))
        for (c, lv, kind, rnd, qo, ql, cb, cc, wb, wc) in rnodes:
            ctx_def = context(p, c, lv)
            for s in ctx_def:
                if s not in cache:
                    raise RuntimeError(f"node ({c},{lv}) in round {t} reads unwritten slot {s}")
            if want is None or (c, lv) in want:
                q = np.asarray(get_q(c, lv), np.float64)
                sel = np.arange(q.shape[0]) if rows is None else np.asarray(rows(c, lv))
                keys = list(cache.keys())
                lens = [cache[s][0].shape[0] for s in keys]
                kall = np.concatenate([cache[s][0] for s in keys], axis=0)
                vall = np.concatenate([cache[s][1] for s in keys], axis=0)
                mask = slot_mask(keys, lens, ctx_def, len(sel))
                hs = range(q.shape[1]) if heads is None else heads
                o = np.zeros((len(sel), q.shape[1], vall.shape[2]))
                lse = np.zeros((q.shape[1], len(sel)))
                for h in hs:
                    oh, lh = masked_attention(q[sel, h, :], kall[:, h, :], vall[:, h, :], mask, scale)
                    o[:, h, :] = oh
                    lse[h, :] = lh
                out[(c, lv)] = (o, lse)
            for s in ctx_def:
                future_reads[s] -= 1
                if future_reads[s] == 0:
                    del cache[s]
        if want is not None and all(k in out for k in want):
            break
    return out
