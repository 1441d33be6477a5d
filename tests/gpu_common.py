"""Helpers shared by the GPU parity tests: run plans through the C ABI and
compare with the oracle.  Inputs come from ``wave_inputs``; expected values
come from ``oracle`` only."""
from __future__ import annotations

import sys

import numpy as np

import block_causal_attention_wave_amd as wv
from oracle import plan as op
from oracle.attention import round_to_bf16
from oracle.rollout import rollout
import wave_inputs as wi

# Tolerances on bf16 inputs: the stated max-abs / mean-abs bounds, plus a
# relative Frobenius bound and an LSE bound (outputs at long context are
# ~1e-2 in magnitude, so absolute bounds alone would pass wrong kernels).
MAX_ABS, MEAN_ABS, REL_FRO, LSE_ABS = 2e-2, 2e-3, 1e-2, 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class HostInputs:
    """Seeded fp32 host tensors for small cases (Q/K/V ~ N(0, sigma^2))."""

    def __init__(self, key, heads, head_dim, chunk_len, cond_len, sigma=1.0, layer=0, policy=0,
                 bf16=False, query_len=0):
        self.bf16 = bf16  # hand the kernels bf16-representable values
        self.QL = query_len or chunk_len
        self.key, self.heads, self.hd = key, heads, head_dim
        self.L, self.C, self.sigma, self.layer, self.policy = chunk_len, cond_len, sigma, layer, policy
        self._cache = {}

    def _get(self, chunk, level, which):
        k = (chunk, level, which)
        if k not in self._cache:
            n = self.QL if which == "q" else (self.C if level == wi.COND_LEVEL else self.L)
            seed = wi.tensor_seed(self.key, self.layer, chunk, level, which, self.policy)
            x = wi.host_normal(seed, (n, self.heads, self.hd), self.sigma)
            self._cache[k] = round_to_bf16(x) if self.bf16 else x
        return self._cache[k]

    def q(self, chunk, level):
        return self._get(chunk, level, "q")

    def kv(self, chunk, level):
        return self._get(chunk, level, "k"), self._get(chunk, level, "v")

    # exact values the kernels consume, widened to fp64 (oracle side)
    def q64(self, chunk, level):
        return round_to_bf16(self.q(chunk, level)).astype(np.float64)

    def kv64(self, chunk, level):
        k, v = self.kv(chunk, level)
        return round_to_bf16(k).astype(np.float64), round_to_bf16(v).astype(np.float64)


def freed_after(plan):
    """{round t: physical slots whose occupant (the logical slot last written
    there) no round after t reads}: the slots a rolling cache may reuse."""
    last = {}
    for t in range(plan.num_rounds):
        for n in plan.round_nodes(t).tolist():
            for (c, lv, _p, _l) in plan.node_ctx(n).tolist():
                last[(c, lv)] = t
    occupant, out = {}, {}
    for t in range(plan.num_rounds):
        for (c, lv, p, _l) in plan.round_writes(t).tolist():
            occupant[p] = (c, lv)
        out[t] = sorted(p for p, key in occupant.items() if last.get(key, -1) <= t)
    return out


def poison_slots(cache, slots):
    """NaN-fill whole physical slots of a cache (K and V^T)."""
    for p in slots:
        cache.k[p].fill_(float("nan"))
        cache.vt[p].fill_(float("nan"))


def gpu_rollout(plan, inputs, device, scale, src_dtype="fp32", poison=True, perturb=None, splits=None,
                balance=True):
    """Run every round of `plan` on the GPU; return {(chunk, level): (O fp32 [L,h,d], LSE [h,L])}.

    perturb(chunk, level, k, v) -> (k, v) may alter the fresh K/V of a slot.
    splits: None = wave_attn, else wave_attn_splitkv with that many splits (0 = auto).
    balance: wave_attn's tail balancing (library's choice for this device).
    poison: the cache starts as NaN, and after every round each slot whose
    occupant no later round reads is NaN-filled again, so a read of a freed
    slot shows up as a non-finite output.
    """
    import torch
    dt = torch.float32 if src_dtype == "fp32" else torch.bfloat16
    desc = plan.upload(device)
    cache = wv.KVCache(plan.num_phys_slots, inputs.heads, inputs.hd, plan.lpad(), device,
                       fill=float("nan") if poison else 0.0)
    outs = {}
    freed = freed_after(plan) if poison else {}
    for t in range(plan.num_rounds):
        ks, vs = [], []
        for (c, lv, _pid, _ln) in plan.round_writes(t).tolist():
            k, v = inputs.kv(c, lv)
            if perturb is not None:
                k, v = perturb(c, lv, k, v)
            ks.append(k)
            vs.append(v)
        k_src = torch.from_numpy(np.concatenate(ks)).to(device=device, dtype=dt)
        v_src = torch.from_numpy(np.concatenate(vs)).to(device=device, dtype=dt)
        wv.kv_write(plan, desc, t, cache, k_src, v_src)
        nodes = plan.round_nodes(t).tolist()
        q = torch.from_numpy(np.concatenate([inputs.q(n[0], n[1]) for n in nodes])).to(device=device, dtype=dt)
        if splits is None:
            o, lse = wv.wave_attn(plan, desc, t, cache, q, scale, balance=balance)
        else:
            o, lse = wv.wave_attn_splitkv(plan, desc, t, cache, q, scale, num_splits=splits)
        torch.cuda.synchronize()
        o = o.float().cpu().numpy()
        lse = lse.cpu().numpy()
        for n in nodes:
            a, b = n[4], n[4] + n[5]
            outs[(n[0], n[1])] = (o[a:b], lse[:, a:b])
        poison_slots(cache, freed.get(t, []))
    return outs


def oracle_rollout(B, K, policy, H, L, cond, inputs, scale, rows=None, heads=None, want=None, query_len=0):
    p = op.Params(B, K, policy, op.SERIAL, H, L, cond, query_len)
    return rollout(p, op.oracle_plan(p), inputs.q64, inputs.kv64, scale, rows=rows, heads=heads,
                   want=want)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o_gpu = np.asarray(o_gpu, np.float64)
    err = np.abs(o_gpu - o_ref)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 rel_fro=float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)),
                 lse_abs=float(np.abs(np.asarray(lse_gpu, np.float64) - lse_ref).max()))
    ok = (stats["max_abs"] <= MAX_ABS and stats["mean_abs"] <= MEAN_ABS and stats["rel_fro"] <= REL_FRO
          and stats["lse_abs"] <= LSE_ABS and np.all(np.isfinite(o_gpu)))
    assert ok, f"{what}: {stats}"
    return stats


def sample_rows(L, n=256, seed=1234, q_tile=256, ragged=True):
    """Deterministic query-row sample: first/last 8 rows, the whole ragged last
    q-tile (when `ragged`), and random rows up to n."""
    rng = np.random.default_rng(seed)
    must = set(range(min(8, L))) | set(range(max(0, L - 8), L))
    last_tile = (L // q_tile) * q_tile
    if ragged and last_tile < L:
        must |= set(range(last_tile, L))
    rest = [r for r in rng.permutation(L).tolist() if r not in must]
    rows = sorted(must | set(rest[:max(0, n - len(must))]))
    return np.asarray(rows)
