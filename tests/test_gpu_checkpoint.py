"""Checkpoint and resume of a rollout.

The whole state of a pipelined rollout between rounds is the round index and
the per-layer K/V cache (every node's query and fresh K/V are inputs of its
round; the plan is rebuilt from its parameters).  Running rounds [0, t),
copying the cache to host memory, restoring it into a freshly allocated
(NaN-filled) cache and running rounds [t, R) must give bitwise the outputs of
the uninterrupted rollout.  Freed slots are NaN-poisoned after every round in
both runs, so a resumed round that read a slot the checkpoint did not carry
would show up as non-finite output.
"""
from __future__ import annotations

import numpy as np
import pytest

import block_causal_attention_wave_amd as wv
import wave_inputs as wi
from gpu_common import HostInputs, freed_after, log, poison_slots

pytestmark = pytest.mark.gpu


def _rounds(plan, inp, desc, cache, rounds, device, scale, splits=None):
    import torch
    freed = freed_after(plan)
    out = {}
    for t in rounds:
        ws = plan.round_writes(t).tolist()
        k = torch.from_numpy(np.concatenate([inp.kv(c, lv)[0] for (c, lv, _, _) in ws])).to(device)
        v = torch.from_numpy(np.concatenate([inp.kv(c, lv)[1] for (c, lv, _, _) in ws])).to(device)
        wv.kv_write(plan, desc, t, cache, k, v)
        nodes = plan.round_nodes(t).tolist()
        q = torch.from_numpy(np.concatenate([inp.q(n[0], n[1]) for n in nodes])).to(device)
        if splits is None:
            o, lse = wv.wave_attn(plan, desc, t, cache, q, scale)
        else:
            o, lse = wv.wave_attn_splitkv(plan, desc, t, cache, q, scale, num_splits=splits)
        torch.cuda.synchronize()
        o, lse = o.cpu(), lse.cpu()
        for n in nodes:
            out[(n[0], n[1])] = (o[n[4]:n[4] + n[5]].clone(), lse[:, n[4]:n[4] + n[5]].clone())
        poison_slots(cache, freed[t])
    return out


@pytest.mark.parametrize("policy,cond,qlen,splits", [(wi.PROGRESSIVE, 0, 0, None), (wi.SAME_LEVEL, 40, 0, None),
                                                      (wi.CLEAN, 0, 0, None), (wi.SAME_LEVEL, 40, 32, 3)])
def test_checkpoint_resume_is_bitwise(gpu_device, policy, cond, qlen, splits):
    import torch
    B, K, L, heads, hd = 6, 3, 300, 2, 128
    plan = wv.wave_plan(B=B, K=K, policy=policy, sched=wv.WAVE, chunk_len=L, cond_len=cond, query_len=qlen)
    inp = HostInputs(500 + policy, heads, hd, L, cond, bf16=True, query_len=qlen)
    scale = 1.0 / np.sqrt(hd)
    desc = plan.upload(gpu_device)
    R = plan.num_rounds

    def fresh():
        return wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), gpu_device, fill=float("nan"))

    full = _rounds(plan, inp, desc, fresh(), range(R), gpu_device, scale, splits)
    for t in sorted({1, R // 2, R - 1}):
        log(f"policy {policy} cond {cond} qlen {qlen}: checkpoint after {t} of {R} rounds")
        c1 = fresh()
        first = _rounds(plan, inp, desc, c1, range(t), gpu_device, scale, splits)
        host_k, host_vt = c1.k.cpu(), c1.vt.cpu()  # the checkpoint
        del c1
        torch.cuda.empty_cache()
        c2 = fresh()
        c2.k.copy_(host_k.to(gpu_device))
        c2.vt.copy_(host_vt.to(gpu_device))
        second = _rounds(plan, inp, desc, c2, range(t, R), gpu_device, scale, splits)
        got = {**first, **second}
        assert set(got) == set(full)
        for key, (o, lse) in full.items():
            assert torch.isfinite(o.float()).all(), key
            assert torch.equal(got[key][0], o) and torch.equal(got[key][1], lse), (t, key)
