"""GPU tests of the toy denoiser chain: qkv_project, chain_store and whole chains.

Expected values come from ``oracle.chain`` only; inputs from ``wave_inputs``.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import block_causal_attention_wave_amd as wv
from oracle import chain as oc
from oracle import plan as op
from oracle.attention import round_to_bf16
import wave_inputs as wi
from gpu_common import log

pytestmark = pytest.mark.gpu


def bf16(x):
    return round_to_bf16(np.asarray(x, np.float32))


def _inputs(key, B, L, heads, hd, layers):
    D = heads * hd
    noise = {c: bf16(wi.host_chain_noise(key, c, L, D)) for c in range(B)}
    weights = [bf16(wi.host_chain_weight(key, l, D)) for l in range(layers)]
    return noise, weights


def gpu_chain(plan, B, L, heads, hd, noise, weights, scale, device, balance=False, fused_rms=True):
    """Run the chain over `plan` on the GPU; return {(chunk, level): [O per layer as [L, heads, hd] fp32]}.

    fused_rms: a layer after the first takes its input rows' RMS from the
    per-head sums of squares that the previous layer's attention wrote with
    its O (wave_attn row_sq), instead of a pass over the rows."""
    import torch
    D = heads * hd
    layers = len(weights)
    desc = plan.upload(device)
    caches = [wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), device, fill=float("nan"))
              for _ in range(layers)]
    w_dev = [torch.from_numpy(w).to(device=device, dtype=torch.bfloat16) for w in weights]
    state = torch.from_numpy(np.stack([noise[c] for c in range(B)])).to(device=device, dtype=torch.bfloat16)
    max_rows = int(plan.round_q_rows.max())
    sq = [torch.full((max_rows, heads), float("nan"), device=device) for _ in range(2)]
    outs = {}
    for t in range(plan.num_rounds):
        rows = int(plan.round_q_rows[t])
        x, layout, x_sq = state, wv.X_CHUNK, None
        per_layer = []
        for layer in range(layers):
            q = wv.qkv_project(plan, desc, t, caches[layer], x, w_dev[layer], x_layout=layout, row_sq=x_sq)
            o_sq = sq[layer & 1] if fused_rms else None
            o, _ = wv.wave_attn(plan, desc, t, caches[layer], q, scale, balance=balance, row_sq=o_sq)
            per_layer.append(o)
            x, layout, x_sq = o.view(rows, D), wv.X_ROUND, o_sq
        wv.chain_store(plan, desc, t, per_layer[-1], state)
        torch.cuda.synchronize()
        for n in plan.round_nodes(t).tolist():
            a, b = n[4], n[4] + n[5]
            outs[(n[0], n[1])] = [o[a:b].float().cpu().numpy() for o in per_layer]
    return outs


@pytest.mark.parametrize("heads,hd,L,layout", [(2, 64, 300, wv.X_CHUNK), (1, 128, 129, wv.X_ROUND),
                                               (3, 128, 200, wv.X_CHUNK), (4, 64, 64, wv.X_ROUND),
                                               (2, 128, 300, wv.X_CHUNK), (4, 128, 520, wv.X_ROUND),
                                               (2, 128, 400, wv.X_ROUND)])
def test_qkv_project_parity(gpu_device, heads, hd, L, layout):
    # D = heads * hd: 128 and 384 take the 128-column kernel, 256 and 512 the
    # 256-column one; L = 300 and 520 give a last row tile of at most 128 slot
    # rows (dispatched last, half its waves idle), L = 400 one of 192 rows.
    """Q, K and V^T of one round against oracle.chain.project on the same bf16
    inputs, slot tails exactly zero, slots of other rounds untouched.  Bound
    per element: one bf16 rounding step (2^-7 relative) on top of the fp32
    summation error of a D-term dot product, gamma * sum_c |a_c w_oc| / rms(a)
    with gamma = D * 2^-24 (the standard worst-case bound for recursive
    summation); the latter matters only where the sum cancels to near zero."""
    import torch
    D = heads * hd
    plan = wv.wave_plan(B=3, K=2, policy=wi.PROGRESSIVE, sched=wv.WAVE, chunk_len=L)
    t = 2  # three nodes: U(0,...), U(1,...) and one more
    nodes = plan.round_nodes(t).tolist()
    rows = int(plan.round_q_rows[t])
    log(f"qkv_project heads={heads} hd={hd} L={L} layout={layout} nodes={[(n[0], n[1]) for n in nodes]}")
    rng = np.random.default_rng(11)
    w = bf16(rng.standard_normal((3 * D, D)) / math.sqrt(D))
    if layout == wv.X_CHUNK:
        x_host = bf16(rng.standard_normal((3, L, D)) * 1.5)
        a_of = {(n[0], n[1]): x_host[n[0]] for n in nodes}
    else:
        x_host = bf16(rng.standard_normal((rows, D)) * 0.7)
        a_of = {(n[0], n[1]): x_host[n[4]:n[4] + n[5]] for n in nodes}
    desc = plan.upload(gpu_device)
    cache = wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), gpu_device, fill=float("nan"))
    x = torch.from_numpy(x_host).to(device=gpu_device, dtype=torch.bfloat16)
    q = wv.qkv_project(plan, desc, t, cache, x, torch.from_numpy(w).to(device=gpu_device, dtype=torch.bfloat16),
                       x_layout=layout)
    torch.cuda.synchronize()
    q = q.float().cpu().numpy()
    k_all = cache.k.float().cpu().numpy()
    vt_all = cache.vt.float().cpu().numpy()
    lpad = plan.lpad()
    written = set()
    for n in nodes:
        a = a_of[(n[0], n[1])].astype(np.float64)
        qo, ko, vo = oc.project(a, w.astype(np.float64), heads, hd)
        inv = 1.0 / np.sqrt(np.mean(a * a, axis=1) + 1e-6)
        acc_err = (D * 2.0 ** -24) * (np.abs(a) @ np.abs(w.astype(np.float64)).T) * inv[:, None]
        acc_q, acc_k, acc_v = (acc_err[:, i * D:(i + 1) * D].reshape(-1, heads, hd) for i in range(3))
        ctx = plan.node_ctx(n)  # own slot last
        phys = int(ctx[-1][2])
        written.add(phys)
        for name, got, ref, acc in (("q", q[n[4]:n[4] + n[5]], qo, acc_q),
                                    ("k", k_all[phys][:, :L].transpose(1, 0, 2), ko, acc_k),
                                    ("v", vt_all[phys][:, :, :L].transpose(2, 0, 1), vo, acc_v)):
            err = np.abs(got - ref)
            bound = 2.0 ** -7 * (np.abs(ref) + acc) + acc
            assert (err <= bound).all(), f"node {(n[0], n[1])} {name}: worst {err.max()}"
        assert (k_all[phys][:, L:] == 0).all() and (vt_all[phys][:, :, L:] == 0).all()
    for s in range(plan.num_phys_slots):
        if s not in written:
            assert np.isnan(k_all[s]).all() and np.isnan(vt_all[s]).all(), f"slot {s} written"


def test_chain_store_copies_node_rows(gpu_device):
    import torch
    L, D = 96, 128
    plan = wv.wave_plan(B=4, K=2, policy=wi.SAME_LEVEL, sched=wv.WAVE, chunk_len=L)
    desc = plan.upload(gpu_device)
    t = 3
    rows = int(plan.round_q_rows[t])
    o = torch.arange(rows * D, device=gpu_device, dtype=torch.float32).remainder(251).to(torch.bfloat16).view(rows, D)
    state = torch.full((4, L, D), -1.0, device=gpu_device, dtype=torch.bfloat16)
    wv.chain_store(plan, desc, t, o, state)
    torch.cuda.synchronize()
    seen = set()
    for n in plan.round_nodes(t).tolist():
        assert torch.equal(state[n[0]], o[n[4]:n[4] + n[5]])
        seen.add(n[0])
    for c in range(4):
        if c not in seen:
            assert (state[c] == -1).all()


@pytest.mark.parametrize("balance", [False, True])
def test_attention_row_sq_feeds_projection(gpu_device, balance):
    """wave_attn's row_sq (wave_attn_chain) against the host sum over head_dim
    of the squares of the bf16 O it returned (fp32 sums of 64 or 128 exact
    squares: relative error below 2^-17), with and without the tail-balancing
    merge kernel writing part of the rows; then qkv_project of the next layer
    taking the RMS from row_sq matches qkv_project taking it from the rows to
    one bf16 step (the two 1/rms differ by a few fp32 roundings), and the
    oracle's projection within its bound."""
    import torch
    heads, hd, L = 4, 128, 520
    D = heads * hd
    plan = wv.wave_plan(B=5, K=3, policy=wi.PROGRESSIVE, sched=wv.WAVE, chunk_len=L)
    t = max(range(plan.num_rounds), key=lambda r: len(plan.round_nodes(r)))
    rows = int(plan.round_q_rows[t])
    nodes = plan.round_nodes(t).tolist()
    log(f"row_sq balance={balance} round {t} rows {rows}")
    rng = np.random.default_rng(5)
    desc = plan.upload(gpu_device)
    cache = wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), gpu_device, fill=0.0)
    for r in range(t + 1):
        n_new = sum(int(wr[3]) for wr in plan.round_writes(r).tolist())
        k = torch.from_numpy(bf16(rng.standard_normal((n_new, heads, hd)))).to(gpu_device, torch.bfloat16)
        v = torch.from_numpy(bf16(rng.standard_normal((n_new, heads, hd)))).to(gpu_device, torch.bfloat16)
        wv.kv_write(plan, desc, r, cache, k, v)
    q = torch.from_numpy(bf16(rng.standard_normal((rows, heads, hd)))).to(gpu_device, torch.bfloat16)
    sq = torch.full((rows, heads), float("nan"), device=gpu_device)
    o, _ = wv.wave_attn(plan, desc, t, cache, q, 1.0 / math.sqrt(hd), balance=balance, row_sq=sq)
    torch.cuda.synchronize()
    o64 = o.float().cpu().numpy().astype(np.float64)
    want = (o64 * o64).sum(axis=2)
    got = sq.cpu().numpy()
    assert np.isfinite(got).all()
    assert np.allclose(got, want, rtol=2.0 ** -17, atol=0.0), float(np.abs(got - want).max())
    # the next layer's projection, RMS from row_sq against RMS from the rows
    w = bf16(rng.standard_normal((3 * D, D)) / math.sqrt(D))
    w_dev = torch.from_numpy(w).to(gpu_device, torch.bfloat16)
    c1 = wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), gpu_device, fill=float("nan"))
    c2 = wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), gpu_device, fill=float("nan"))
    x = o.view(rows, D)
    q1 = wv.qkv_project(plan, desc, t, c1, x, w_dev, x_layout=wv.X_ROUND, row_sq=sq)
    q2 = wv.qkv_project(plan, desc, t, c2, x, w_dev, x_layout=wv.X_ROUND)
    torch.cuda.synchronize()
    for a, b in ((q1, q2), (c1.k, c2.k), (c1.vt, c2.vt)):
        a, b = a.float().cpu().numpy(), b.float().cpu().numpy()
        assert np.array_equal(np.isnan(a), np.isnan(b))
        a, b = np.nan_to_num(a), np.nan_to_num(b)
        assert (np.abs(a - b) <= 2.0 ** -7 * np.abs(b)).all()
    q1 = q1.float().cpu().numpy()
    for n in nodes:
        a = o64[n[4]:n[4] + n[5]].reshape(n[5], D)
        qo, _, _ = oc.project(a, w.astype(np.float64), heads, hd)
        inv = 1.0 / np.sqrt(np.mean(a * a, axis=1) + 1e-6)
        acc = ((D * 2.0 ** -24) * (np.abs(a) @ np.abs(w.astype(np.float64)).T) * inv[:, None])[:, :D]
        acc = acc.reshape(n[5], heads, hd)
        err = np.abs(q1[n[4]:n[4] + n[5]] - qo)
        assert (err <= 2.0 ** -7 * (np.abs(qo) + acc) + acc).all(), (n[0], n[1])


CHAIN_GRID = [
    # policy, B, K, L, heads, hd, layers
    (wi.PROGRESSIVE, 3, 2, 160, 2, 64, 2),
    (wi.SAME_LEVEL, 4, 2, 130, 1, 128, 1),
    (wi.CLEAN, 3, 3, 96, 2, 64, 2),
    (wi.PROGRESSIVE, 3, 2, 200, 4, 64, 2),
]


@pytest.mark.parametrize("fused_rms", [True, False])
@pytest.mark.parametrize("policy,B,K,L,heads,hd,layers", CHAIN_GRID)
def test_chain_matches_oracle(gpu_device, policy, B, K, L, heads, hd, layers, fused_rms):
    """Every node's per-layer attention output of a whole chain against the
    independent fp64 chain oracle, with the RMS of a layer's input taken from
    the previous attention's per-head sums of squares or from the rows."""
    noise, weights = _inputs(40 + L, B, L, heads, hd, layers)
    scale = 1.0 / math.sqrt(hd)
    plan = wv.wave_plan(B=B, K=K, policy=policy, sched=wv.WAVE, chunk_len=L)
    log(f"chain policy={policy} B={B} K={K} L={L} heads={heads} hd={hd} layers={layers} fused_rms={fused_rms}")
    got = gpu_chain(plan, B, L, heads, hd, noise, weights, scale, gpu_device, fused_rms=fused_rms)
    p = op.Params(B, K, policy, op.SERIAL, -1, L, 0, 0)
    ref = oc.chain_rollout(p, op.oracle_plan(p), layers, heads, hd, lambda c: noise[c].astype(np.float64),
                           lambda l: weights[l].astype(np.float64), scale)
    assert set(got) == set(ref)
    worst = 0.0
    for key, (_, per_layer) in ref.items():
        for layer, (g, r) in enumerate(zip(got[key], per_layer)):
            rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
            worst = max(worst, rel)
            assert np.isfinite(g).all()
            assert rel <= CHAIN_REL_FRO, f"node {key} layer {layer}: rel {rel}"
    log(f"  worst relative Frobenius error {worst:.3g}")


# Bound for whole chains, relative Frobenius norm per node and layer.  One
# stage (projection, then attention) adds at most e = 3e-3: two bf16 roundings
# (Q/K/V and O, each 2^-9 relative at worst, about 2^-9/sqrt(3) in RMS) plus
# the attention's own fp32/bf16 error (about 1e-3 at these sizes).  An input
# error grows by at most g = 1.5 through a stage: the projection is
# RMS-normalised, and the softmax of unit-variance scaled scores changes its
# weights by at most about half the relative change of the scores.  The
# deepest stage in CHAIN_GRID is the 6th (3 levels x 2 layers), so
# e * (g^6 - 1) / (g - 1) = 6.2e-2.
CHAIN_REL_FRO = 6e-2


# Bound for one stage (projection, then attention) on exact inputs, relative
# Frobenius norm per node and layer.  Both sides round O to bf16 (unit
# roundoff u = 2^-8: 8 significand bits), the kernel from its fp32 result and
# the oracle from fp64.  The two roundings agree except where the pre-rounding
# values straddle a rounding boundary, and then differ by one bf16 step
# (2^-8 to 2^-7 relative).  The kernel's pre-rounding error is about
# d = 1e-3 relative (bf16 P, fp32 sums), so a fraction of about d / 2^-8 =
# 0.26 of the elements straddle: sqrt(0.26) * 2^-7.5 = 2.8e-3 in RMS, with d
# in quadrature about 3.0e-3.  Q, K and V are rounded to bf16 from an fp32 sum
# on the GPU and an fp64 sum in the oracle; the few elements that land one
# step apart add well under 1e-3.  Bound: 4e-3 (measured worst 2.9e-3).
STAGE_REL_FRO = 4e-3


@pytest.mark.parametrize("policy,B,K,L,heads,hd,layers", CHAIN_GRID)
def test_chain_each_stage_matches_oracle(gpu_device, policy, B, K, L, heads, hd, layers):
    """One stage at a time: every round and layer of the chain runs on the GPU
    (qkv_project into the layer's cache, then wave_attn) with the oracle's own
    input rows for that layer (the noise, or the oracle's output of the
    previous layer or of the chunk's previous node), so each output carries
    the error of a single stage and is held to the one-stage bound instead of
    the compounded whole-chain bound."""
    import torch
    noise, weights = _inputs(40 + L, B, L, heads, hd, layers)
    scale = 1.0 / math.sqrt(hd)
    D = heads * hd
    p = op.Params(B, K, policy, op.SERIAL, -1, L, 0, 0)
    ref = oc.chain_rollout(p, op.oracle_plan(p), layers, heads, hd, lambda c: noise[c].astype(np.float64),
                           lambda l: weights[l].astype(np.float64), scale)
    plan = wv.wave_plan(B=B, K=K, policy=policy, sched=wv.WAVE, chunk_len=L)
    log(f"chain stages policy={policy} B={B} K={K} L={L} heads={heads} hd={hd} layers={layers}")
    # the oracle's input rows of every node at every layer
    prev = {}
    for n in plan.nodes.tolist():  # nodes in round order; a chunk's nodes in execution order
        prev[(n[0], n[1])] = prev.get(("last", n[0]))
        prev[("last", n[0])] = (n[0], n[1])

    def a_in(key, layer):
        if layer > 0:
            return ref[key][1][layer - 1].reshape(L, D)
        return noise[key[0]] if prev[key] is None else ref[prev[key]][0]

    desc = plan.upload(gpu_device)
    caches = [wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), gpu_device, fill=float("nan"))
              for _ in range(layers)]
    w_dev = [torch.from_numpy(w).to(device=gpu_device, dtype=torch.bfloat16) for w in weights]
    worst = 0.0
    for t in range(plan.num_rounds):
        nodes = plan.round_nodes(t).tolist()
        for layer in range(layers):
            x = np.concatenate([a_in((n[0], n[1]), layer) for n in nodes]).astype(np.float32)
            x = torch.from_numpy(x).to(device=gpu_device, dtype=torch.bfloat16)
            q = wv.qkv_project(plan, desc, t, caches[layer], x, w_dev[layer], x_layout=wv.X_ROUND)
            o, _ = wv.wave_attn(plan, desc, t, caches[layer], q, scale, balance=False)
            torch.cuda.synchronize()
            o = o.float().cpu().numpy()
            for n in nodes:
                g = o[n[4]:n[4] + n[5]]
                r = ref[(n[0], n[1])][1][layer]
                rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
                worst = max(worst, rel)
                assert np.isfinite(g).all()
                assert rel <= STAGE_REL_FRO, f"round {t} node {(n[0], n[1])} layer {layer}: rel {rel}"
    log(f"  worst one-stage relative Frobenius error {worst:.3g}")


@pytest.mark.parametrize("policy", [wi.CLEAN, wi.SAME_LEVEL, wi.PROGRESSIVE])
def test_chain_serial_equals_wave_bitwise(gpu_device, policy):
    """Real data flow through the schedule: serial and pipelined rounds give
    bitwise identical outputs for every node and layer."""
    B, K, L, heads, hd, layers = 4, 3, 200, 2, 64, 2
    noise, weights = _inputs(77, B, L, heads, hd, layers)
    outs = {}
    for sched in (wv.SERIAL, wv.WAVE):
        plan = wv.wave_plan(B=B, K=K, policy=policy, sched=sched, chunk_len=L)
        outs[sched] = gpu_chain(plan, B, L, heads, hd, noise, weights, 0.125, gpu_device)
    assert set(outs[wv.SERIAL]) == set(outs[wv.WAVE])
    for key in outs[wv.WAVE]:
        for a, b in zip(outs[wv.SERIAL][key], outs[wv.WAVE][key]):
            assert np.array_equal(a, b), key


def _device_chain(plan, w, layers, device, policy):
    """Full-size chain on the device; returns {(chunk, level): last-layer O (bf16, on the device)}."""
    import torch
    D = w.heads * w.head_dim
    desc = plan.upload(device)
    caches = [wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, plan.lpad(), device, fill=float("nan"))
              for _ in range(layers)]
    weights = [wi.device_chain_weight(w.key, l, D, device) for l in range(layers)]
    state = torch.stack([wi.device_chain_noise(w.key, c, w.chunk_len, D, device) for c in range(w.B)])
    sq = [torch.empty((int(plan.round_q_rows.max()), w.heads), device=device) for _ in range(2)]
    outs = {}
    for t in range(plan.num_rounds):
        rows = int(plan.round_q_rows[t])
        x, layout, x_sq = state, wv.X_CHUNK, None
        for layer in range(layers):
            q = wv.qkv_project(plan, desc, t, caches[layer], x, weights[layer], x_layout=layout, row_sq=x_sq)
            o, _ = wv.wave_attn(plan, desc, t, caches[layer], q, w.scale, want_lse=False, balance=False,
                                row_sq=sq[layer & 1])
            x, layout, x_sq = o.view(rows, D), wv.X_ROUND, sq[layer & 1]
        wv.chain_store(plan, desc, t, o, state)
        for n in plan.round_nodes(t).tolist():
            outs[(n[0], n[1])] = o[n[4]:n[4] + n[5]].clone()
    torch.cuda.synchronize()
    return outs


def test_chain_full_size_serial_equals_wave(gpu_device):
    """The 832x480 seven-chunk K=5 shape (4680 tokens, 12 heads x 128), two
    layers, progressive: serial (35 rounds) and pipelined (11 rounds) chains
    give bitwise identical outputs for every node."""
    import torch
    w = wi.WORKLOADS[3]
    outs = {}
    for sched in (wv.SERIAL, wv.WAVE):
        plan = wv.wave_plan(B=w.B, K=w.K, policy=wi.PROGRESSIVE, sched=sched, chunk_len=w.chunk_len)
        log(f"full-size chain, sched={sched}: {plan.num_rounds} rounds")
        outs[sched] = _device_chain(plan, w, 2, gpu_device, wi.PROGRESSIVE)
    assert set(outs[wv.SERIAL]) == set(outs[wv.WAVE]) and len(outs[wv.WAVE]) >= w.B * w.K
    for key, o in outs[wv.WAVE].items():
        assert torch.equal(o, outs[wv.SERIAL][key]), key
        assert torch.isfinite(o.float()).all()


def test_qkv_project_full_size_sampled(gpu_device):
    """qkv_project of the 832x480 K=4 round 6 (5 nodes x 4680 tokens, D = 1536)
    on the chunks' seeded noise: 48 sampled rows of every node against
    oracle.chain.project, and every written slot's tail exactly zero."""
    import torch
    w = wi.WORKLOADS[2]
    D = w.heads * w.head_dim
    plan = wv.wave_plan(B=w.B, K=w.K, policy=wi.PROGRESSIVE, sched=wv.WAVE, chunk_len=w.chunk_len)
    desc = plan.upload(gpu_device)
    cache = wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, plan.lpad(), gpu_device, fill=float("nan"))
    state = torch.stack([wi.device_chain_noise(w.key, c, w.chunk_len, D, gpu_device) for c in range(w.B)])
    wt = wi.device_chain_weight(w.key, 0, D, gpu_device)
    q = wv.qkv_project(plan, desc, w.round, cache, state, wt, x_layout=wv.X_CHUNK)
    torch.cuda.synchronize()
    w64 = wt.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(3)
    for n in plan.round_nodes(w.round).tolist():
        rows = np.unique(np.concatenate([[0, w.chunk_len - 1], rng.integers(0, w.chunk_len, 46)]))
        a = state[n[0]][rows].float().cpu().numpy().astype(np.float64)
        qo, ko, vo = oc.project(a, w64, w.heads, w.head_dim)
        inv = 1.0 / np.sqrt(np.mean(a * a, axis=1) + 1e-6)
        acc = (D * 2.0 ** -24) * (np.abs(a) @ np.abs(w64).T) * inv[:, None]
        phys = int(plan.node_ctx(n)[-1][2])
        got_q = q[n[4] + rows].float().cpu().numpy()
        got_k = cache.k[phys][:, rows].float().cpu().numpy().transpose(1, 0, 2)
        got_v = cache.vt[phys][:, :, rows].float().cpu().numpy().transpose(2, 0, 1)
        for i, (got, ref) in enumerate(((got_q, qo), (got_k, ko), (got_v, vo))):
            ac = acc[:, i * D:(i + 1) * D].reshape(len(rows), w.heads, w.head_dim)
            assert (np.abs(got - ref) <= 2.0 ** -7 * (np.abs(ref) + ac) + ac).all(), (n[0], n[1], "qkv"[i])
        lp = plan.lpad()
        assert (cache.k[phys][:, w.chunk_len:lp] == 0).all() and (cache.vt[phys][:, :, w.chunk_len:lp] == 0).all()
