"""Brute-force reference planner (TEST INFRASTRUCTURE ONLY; see ``oracle``).

What it computes, and where the pages fix it
--------------------------------------------
* Context policies.  In the streaming-video-diffusion design-space paper
  (thelatestinai.com listing of arXiv 2609.22283), Figure 1 lays the history
  out as a grid of chunks (columns) by denoising levels (rows), and Table 1
  names three policies for the level of the history state read at chunk
  distance r by an update at level j: clean reads level 0, same-level reads
  level j, progressive reads level max(j - r, 0).
* Schedules.  Figure 2 of the same paper: serial execution finishes all K
  updates of one chunk before the next chunk starts (B*K rounds); pipelined
  execution runs chunks at staggered levels (B+K-1 rounds) with the same B*K
  chunk-level updates.
* Refresh.  The Wave Forcing pages (aiany.app summary, opening paragraph and
  Key Findings; aipulsen.com article, second paragraph) describe refreshing a
  finished chunk's history cache as a forward pass of its own.
* Block causality.  The aipulsen.com article (third paragraph) says the
  design has no reverse dependencies across chunks; Wan-Streamer v0.2
  (abstract; "Model Formulation and Upgrade") puts every modality on one
  block-causal timeline and feeds language/state to the generator only as a
  K/V slice.

Readings where the pages are silent
-----------------------------------
* Level 0 is the clean (fully denoised) state, level K pure noise.  Update
  U(i, j) consumes chunk i at level j (j = K..1) and writes the K/V slot
  (i, j).  The clean slot (i, 0) exists only after a refresh node R(i), which
  is created iff some node reads (i, 0).
* History at distance r = 1..min(i, H) (H = -1: unlimited) in timeline order
  (oldest first); each history chunk's conditioning slot C precedes its
  latent slot; the node's own C and its own slot come last.
* Pipelined rounds: a node may read a slot written in an earlier round, or in
  the same round by a lower chunk (all of a round's K/V writes land before its
  attention).  Chunk i is admitted no earlier than round i.  Each chunk runs
  at most one node per round.  Nodes of a round are ordered by chunk.
* Serial rounds: U(i, j) runs in round i*K + K - j; R(i-1) shares round i*K
  with U(i, K).
* Physical slots: a slot is free from the first round after its last reader;
  each write takes the lowest free id, in node order, conditioning first.
"""
from __future__ import annotations

from dataclasses import dataclass

CLEAN, SAME_LEVEL, PROGRESSIVE = 0, 1, 2
SERIAL, WAVE = 0, 1
UPDATE, REFRESH = 0, 1
COND = -1  # level tag of a conditioning (K/V-only) slot


@dataclass(frozen=True)
class Params:
    B: int                 # number of chunks
    K: int                 # number of denoising levels (updates per chunk)
    policy: int            # CLEAN / SAME_LEVEL / PROGRESSIVE
    sched: int             # SERIAL / WAVE
    history_cap: int = -1  # H: history window in chunks, -1 = unlimited
    chunk_len: int = 1     # tokens per chunk (query rows and latent slot length)
    cond_len: int = 0      # tokens of each chunk's conditioning slot, 0 = none
    query_len: int = 0     # query rows per node, 0 = chunk_len (fewer: decode-shaped)


def phi(policy: int, j: int, r: int) -> int:
    """Level of the history state at chunk distance r read by a level-j update.

    Table 1 of the arXiv 2609.22283 listing: clean 0, same-level j,
    progressive max(j - r, 0).
    """
    if policy == CLEAN:
        return 0
    if policy == SAME_LEVEL:
        return j
    if policy == PROGRESSIVE:
        return max(j - r, 0)
    raise ValueError(f"unknown policy {policy}")


def context(p: Params, chunk: int, level: int) -> list[tuple[int, int]]:
    """Logical slots read by the node that computes `chunk` at `level`.

    level >= 1 is an update, level 0 a refresh (phi(., 0, r) is 0 for every
    policy, so a refresh reads clean history).  Returns (chunk, level) pairs,
    level COND for conditioning slots, in timeline order, own slot last.
    """
    window = chunk if p.history_cap < 0 else min(chunk, p.history_cap)
    refs: list[tuple[int, int]] = []
    for r in range(window, 0, -1):
        c = chunk - r
        if p.cond_len > 0:
            refs.append((c, COND))
        refs.append((c, phi(p.policy, level, r)))
    if p.cond_len > 0:
        refs.append((chunk, COND))
    refs.append((chunk, level))
    return refs


@dataclass
class Node:
    chunk: int
    level: int
    kind: int
    ctx: list
    writes: list
    round: int = -1


def build_nodes(p: Params) -> dict[int, list[Node]]:
    """Per chunk, its nodes in execution order: U(i,K) .. U(i,1) [, R(i)]."""
    per_chunk: dict[int, list[Node]] = {}
    for i in range(p.B):
        lst = []
        for j in range(p.K, 0, -1):
            writes = []
            if j == p.K and p.cond_len > 0:
                writes.append((i, COND))
            writes.append((i, j))
            lst.append(Node(i, j, UPDATE, context(p, i, j), writes))
        per_chunk[i] = lst
    # Refresh nodes, to a fixpoint: R(i) exists iff some node reads (i, 0).
    has_refresh: set[int] = set()
    changed = True
    while changed:
        changed = False
        for i in range(p.B):
            for n in per_chunk[i]:
                for (c, lv) in n.ctx:
                    if lv == 0 and (c, lv) not in n.writes and c not in has_refresh:
                        has_refresh.add(c)
                        changed = True
                        per_chunk[c].append(Node(c, 0, REFRESH, context(p, c, 0), [(c, 0)]))
    return per_chunk


def _schedule_wave(p: Params, per_chunk: dict[int, list[Node]]) -> int:
    """As-soon-as-possible round assignment by simulating rounds one by one."""
    pending = {i: list(per_chunk[i]) for i in range(p.B)}
    written: dict[tuple[int, int], int] = {}
    last_round = {i: -1 for i in range(p.B)}
    total = sum(len(v) for v in pending.values())
    t = 0
    limit = 4 * (p.B + 1) * (p.K + 2)
    placed = 0
    while placed < total:
        if t > limit:
            raise RuntimeError("wave schedule did not converge")
        for i in range(p.B):
            if not pending[i] or t < i or last_round[i] >= t:
                continue
            n = pending[i][0]
            ok = True
            for s in n.ctx:
                if s in n.writes:
                    continue
                if s not in written or written[s] > t:
                    ok = False
                    break
            if not ok:
                continue
            n.round = t
            for s in n.writes:
                written[s] = t
            last_round[i] = t
            pending[i].pop(0)
            placed += 1
        t += 1
    return max(n.round for lst in per_chunk.values() for n in lst) + 1


def _schedule_serial(p: Params, per_chunk: dict[int, list[Node]]) -> int:
    for i in range(p.B):
        for n in per_chunk[i]:
            if n.kind == UPDATE:
                n.round = i * p.K + p.K - n.level
            else:
                n.round = (i + 1) * p.K
    return p.B * p.K


def check_legal(per_chunk: dict[int, list[Node]]) -> None:
    """Every read slot was written in an earlier round, or earlier in the same
    round by a lower chunk; a chunk's nodes run in order, one per round."""
    writer: dict[tuple[int, int], Node] = {}
    for lst in per_chunk.values():
        for n in lst:
            for s in n.writes:
                assert s not in writer, f"slot {s} written twice"
                writer[s] = n
    for lst in per_chunk.values():
        for a, b in zip(lst, lst[1:]):
            assert a.round < b.round, "chunk nodes out of order"
        for n in lst:
            for s in n.ctx:
                if s in n.writes:
                    continue
                w = writer.get(s)
                assert w is not None, f"slot {s} read but never written"
                assert w.round < n.round or (w.round == n.round and w.chunk < n.chunk), \
                    f"illegal read of {s} by ({n.chunk},{n.level}) in round {n.round}"


def oracle_plan(p: Params) -> dict:
    """Plan as plain Python lists, in the same field order as the C view."""
    if p.B <= 0 or p.K <= 0 or p.policy not in (0, 1, 2) or p.sched not in (0, 1):
        raise ValueError("invalid params")
    per_chunk = build_nodes(p)
    num_rounds = _schedule_wave(p, per_chunk) if p.sched == WAVE else _schedule_serial(p, per_chunk)
    check_legal(per_chunk)

    rounds: list[list[Node]] = [[] for _ in range(num_rounds)]
    for i in range(p.B):
        for n in per_chunk[i]:
            rounds[n.round].append(n)
    for r in rounds:
        r.sort(key=lambda n: n.chunk)

    def slot_len(s):
        return p.cond_len if s[1] == COND else p.chunk_len

    # Liveness: last round that reads each slot.
    last_read: dict[tuple[int, int], int] = {}
    for t, r in enumerate(rounds):
        for n in r:
            for s in n.ctx:
                last_read[s] = max(last_read.get(s, -1), t)

    phys: dict[tuple[int, int], int] = {}
    in_use: dict[int, tuple[int, int]] = {}
    capacity = 0
    for t, r in enumerate(rounds):
        for pid, s in list(in_use.items()):
            if last_read[s] < t:
                del in_use[pid]
        for n in r:
            for s in n.writes:
                pid = 0
                while pid in in_use:
                    pid += 1
                in_use[pid] = s
                phys[s] = pid
                capacity = max(capacity, pid + 1)

    q_len = p.query_len if p.query_len > 0 else p.chunk_len
    round_node_begin = [0]
    nodes, ctx, writes = [], [], []
    for t, r in enumerate(rounds):
        q_off = 0
        for n in r:
            nodes.append((n.chunk, n.level, n.kind, t, q_off, q_len,
                          len(ctx), len(n.ctx), len(writes), len(n.writes)))
            q_off += q_len
            for s in n.ctx:
                ctx.append((s[0], s[1], phys[s], slot_len(s)))
            for s in n.writes:
                writes.append((s[0], s[1], phys[s], slot_len(s)))
        round_node_begin.append(len(nodes))
    return {
        "num_rounds": num_rounds,
        "num_phys_slots": capacity,
        "round_node_begin": round_node_begin,
        "nodes": nodes,
        "ctx": ctx,
        "writes": writes,
    }
