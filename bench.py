#!/usr/bin/env python3
"""Benchmark of one pipelined wave round of block-causal attention on one MI355X.

A step is one pass of the round's device path: ``kv_write`` of the round's
fresh K/V into the cache, then ``wave_attn`` of every query chunk in flight.
The plan (host) is built once before timing: one plan serves every round and
every layer of a rollout; its host cost is reported as ``plan_ms``.

Default workload: the Wan2.1-T2V-1.3B 832x480 shape (12 heads x 128, 4680
tokens per 3-latent-frame chunk, 7 chunks), K=4 levels, progressive history,
pipelined round 6: R(2), U(3,1), U(4,2), U(5,3), U(6,4) over 32,760 keys.

Prints ONE JSON line on stdout.  Extra flags:
  --rollout              whole rollouts instead of one round: workload 3 (7 chunks, K=5,
                         30 layers, clean / same-level / progressive) or 4 (28 chunks, K=4,
                         history cap 6); every (round, layer) runs kv_write + wave_attn, each
                         pair timed with events after its inputs are generated
  --workload {2,4,5,6}   2 (default), 4 = long video steady round, 5 = Wan-Streamer round,
                         6 = Wan-Streamer audio decode (64 query rows per chunk, split-KV)
  --no-cpu-baseline      skip the CPU oracle timing
  --copy-calibration     also run one 1 GiB device copy (HBM counter calibration)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_flops(plan, t, heads, head_dim, rows_per_node=None):
    """4 * heads * d * sum over nodes of (query rows x unmasked keys)."""
    total = 0
    for n in plan.round_nodes(t):
        keys = int(plan.node_ctx(n)[:, 3].sum())
        rows = int(n[5]) if rows_per_node is None else rows_per_node
        total += rows * keys
    return 4.0 * heads * head_dim * total


def kv_write_bytes(plan, t, heads, head_dim, lpad, src_bytes=2):
    """Read fresh K and V (len rows) + write K and V^T slots (lpad rows each, tail zeroed)."""
    b = 0
    for w in plan.round_writes(t):
        b += 2 * int(w[3]) * heads * head_dim * src_bytes
        b += 2 * lpad * heads * head_dim * 2
    return b


HBM_PROFILES = {2: "wave_attn_wan13b_round6_hbm.md", 4: "wave_attn_longvideo_round16_hbm.md",
                5: "wave_attn_streamer_round7_hbm.md", 6: "wave_attn_streamer_audio_decode_hbm.md"}


def traffic_from_profile(workload):
    """HBM bytes per wave_attn launch from the committed rocprofv3 counter
    summary, or None if there is none or the kernel source changed since."""
    import hashlib
    name = HBM_PROFILES.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for src in fields["kernel_sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["kernel_source_sha256"]:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def attention_bytes(plan, t, heads, head_dim):
    """Compulsory HBM bytes of one round's attention: Q and O (bf16), the LSE,
    and each distinct cache slot the round's gather lists read (K and V)."""
    slots = {}
    rows = 0
    for n in plan.round_nodes(t):
        rows += int(n[5])
        for c in plan.node_ctx(n):
            slots[(int(c[0]), int(c[1]))] = int(c[3])
    kv = sum(slots.values()) * heads * head_dim * 2 * 2
    return kv + rows * heads * head_dim * 2 * 2 + rows * heads * 4


def sample_rows(L, n, seed=1234):
    rng = np.random.default_rng(seed)
    must = set(range(min(8, L))) | set(range(max(0, L - 8), L))
    rest = [r for r in rng.permutation(L).tolist() if r not in must]
    return np.asarray(sorted(must | set(rest[:max(0, n - len(must))])))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=(1, 2, 3, 4, 5, 6))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768,
                    help="query rows per node for the CPU oracle (bounded sample, ~10-30 s of CPU work)")
    ap.add_argument("--splits", type=int, default=0,
                    help="split-KV key ranges for decode-shaped rounds (0 = the library's choice)")
    ap.add_argument("--no-balance", action="store_true",
                    help="wave_attn without tail balancing (each node bitwise independent of the schedule)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--rollout", action="store_true")
    ap.add_argument("--chain", action="store_true",
                    help="whole rollouts of the toy denoiser chain (QKV projection into the cache + attention)")
    ap.add_argument("--proj", action="store_true",
                    help="qkv_project against the plain bf16 product (torch.matmul) of the same shape, "
                         "one round per node count of the Wan2.1-1.3B pipelined plan")
    ap.add_argument("--layers", type=int, default=0, help="rollout layers (0 = the workload's)")
    ap.add_argument("--no-fused-rms", action="store_true",
                    help="with --chain, take each layer's input RMS from a pass over its rows instead of "
                         "from the per-head sums of squares the previous attention wrote")
    ap.add_argument("--no-extra", action="store_true",
                    help="with workload 2, skip the Wan-Streamer round and audio decode timed after it")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(no collectives, no sharding); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_causal_attention_wave_amd as wv
    import wave_inputs as wi

    device = torch.device("cuda:0")
    if args.chain:
        chain_bench(args, device)
        return
    if args.proj:
        proj_bench(args, device)
        return
    if args.rollout:
        rollout_bench(args, device)
        return
    if args.workload == 3:
        print("workload 3 is a whole rollout: run it with --rollout", file=sys.stderr)
        sys.exit(2)
    if args.workload == 1:
        tiny_bench(args, device)
        return
    out = measure_round(args, device, args.workload, args.steps, args.warmup, cpu=not args.no_cpu_baseline,
                        copy_calibration=args.copy_calibration)
    if args.workload == 2 and not args.no_extra:
        # The Wan-Streamer-shaped round and its audio decode, timed in the same run.
        extra = {}
        for key in (5, 6):
            r = measure_round(args, device, key, max(10, args.steps // 2), max(3, args.warmup // 2), cpu=False,
                              copy_calibration=False)
            extra[r["config"]["workload"]] = {
                "metric": r["roofline"]["unit"], "achieved": r["roofline"]["achieved"],
                "frac_of_peak": r["roofline"]["frac"], "bound": r["roofline"]["bound"],
                "attn_ms": r["attn_ms"], "attn_ms_median": r["attn_ms_median"], "round_ms": r["round_ms"],
                "kv_write_ms": r["kv_write_ms"], "kv_write_gbps": r["kv_write_gbps"],
                "algorithmic_tflop": r["config"]["algorithmic_tflop"], "attn_compulsory_mb": r["attn_compulsory_mb"],
                "splitkv_splits": r["config"]["splitkv_splits"], "traffic": r["roofline"]["traffic"],
                "steps": r["steps"]}
        out["extra_workloads"] = extra
    print(json.dumps(out), flush=True)


def measure_round(args, device, key, steps, warmup, cpu, copy_calibration):
    """kv_write + wave_attn of one round of workload `key`, timed over `steps`
    steps after `warmup`; returns the bench JSON object (without printing it)."""
    import torch
    import block_causal_attention_wave_amd as wv
    import wave_inputs as wi

    w = wi.WORKLOADS[key]
    policy = w.policies[0]
    t_meas = w.round if w.round >= 0 else 16
    layer = 0

    t0 = time.perf_counter()
    plan = wv.wave_plan(B=w.B, K=w.K, policy=policy, sched=wv.WAVE, chunk_len=w.chunk_len,
                        cond_len=w.cond_len, history_cap=w.history_cap, query_len=w.query_len)
    decode = w.query_len > 0
    plan_ms = (time.perf_counter() - t0) * 1e3
    desc = plan.upload(device)
    lpad = plan.lpad()
    cache = wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, lpad, device, fill=float("nan"))

    # Prefill: the earlier rounds' K/V writes (their attention is not needed).
    def fresh(t):
        ws = plan.round_writes(t).tolist()
        ks = [wi.device_tensor(w, layer, c, lv, "k", device, policy) for (c, lv, _, _) in ws]
        vs = [wi.device_tensor(w, layer, c, lv, "v", device, policy) for (c, lv, _, _) in ws]
        return torch.cat(ks), torch.cat(vs)

    for t in range(t_meas):
        k_src, v_src = fresh(t)
        wv.kv_write(plan, desc, t, cache, k_src, v_src)
    k_src, v_src = fresh(t_meas)
    nodes = plan.round_nodes(t_meas).tolist()
    qlen = w.query_len or w.chunk_len
    # decode-shaped: the last query_len tokens of each chunk (its audio latents)
    q = torch.cat([wi.device_tensor(w, layer, n[0], n[1], "q", device, policy)[-qlen:] for n in nodes])
    rows = int(plan.round_q_rows[t_meas])
    o = torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=device)
    lse = torch.empty((w.heads, rows), dtype=torch.float32, device=device)
    torch.cuda.synchronize()

    flops = algorithmic_flops(plan, t_meas, w.heads, w.head_dim)
    kvw_bytes = kv_write_bytes(plan, t_meas, w.heads, w.head_dim, lpad)
    attn_bytes = attention_bytes(plan, t_meas, w.heads, w.head_dim)
    workspace = None
    splits = 1
    tail = (0, 1)
    if decode:
        nbytes, splits = wv.splitkv_workspace_bytes(plan, t_meas, w.heads, w.head_dim, args.splits)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif not args.no_balance:
        # tail balancing: the library's choice of trailing work items to cut
        nbytes, tail_items, tail_splits = wv.attn_workspace(plan, t_meas, w.heads, w.head_dim)
        tail = (tail_items, tail_splits)
        if nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def attn(stream):
        if decode:
            return wv.wave_attn_splitkv(plan, desc, t_meas, cache, q, w.scale, num_splits=splits,
                                        workspace=workspace, o=o, lse=lse, stream=stream)
        return wv.wave_attn(plan, desc, t_meas, cache, q, w.scale, o=o, lse=lse, stream=stream,
                            balance=not args.no_balance, workspace=workspace)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            wv.kv_write(plan, desc, t_meas, cache, k_src, v_src, stream=stream)
            attn(stream)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1, e2 in evs:
            e0.record(stream)
            wv.kv_write(plan, desc, t_meas, cache, k_src, v_src, stream=stream)
            e1.record(stream)
            attn(stream)
            e2.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    kvw_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    attn_ms = np.array([b.elapsed_time(c) for _, b, c in evs])
    if not torch.isfinite(o.float()).all() or not torch.isfinite(lse).all():
        eprint("non-finite output: a read outside the written slots")
        sys.exit(3)

    ms_per_step = wall * 1e3 / steps
    attn_avg = float(attn_ms.mean())
    achieved = flops / (attn_avg * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_gbps = attn_bytes / (attn_avg * 1e-3) / 1e9
    eprint(f"[bench] {w.name}: round {t_meas}, {len(nodes)} nodes, {rows} query rows, "
           f"{flops / 1e12:.3f} TFLOP")
    eprint(f"[bench] wave_attn {attn_avg:.3f} ms (p10 {np.percentile(attn_ms, 10):.3f}, "
           f"p90 {np.percentile(attn_ms, 90):.3f}) = {achieved:.1f} TFLOP/s = "
           f"{100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")
    eprint(f"[bench] wave_attn moves {attn_bytes / 1e6:.1f} MB compulsory = {attn_gbps:.0f} GB/s"
           + (f" (split-KV, {splits} splits)" if decode else ""))
    eprint(f"[bench] kv_write {kvw_ms.mean() * 1e3:.1f} us = {kvw_bytes / (kvw_ms.mean() * 1e-3) / 1e9:.0f} GB/s; "
           f"step {ms_per_step:.3f} ms wall")

    copy_ms = None
    if copy_calibration:
        n = 1 << 29  # 1 GiB of bf16
        src = torch.ones(n, dtype=torch.bfloat16, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_ms = e0.elapsed_time(e1)
        eprint(f"[bench] 1 GiB copy {copy_ms:.3f} ms = {2 * (1 << 30) / (copy_ms * 1e-3) / 1e9:.0f} GB/s")
        del src, dst

    cpu_res = None
    if cpu:
        cpu_res = cpu_baseline(w, plan, t_meas, nodes, policy, layer, device, args.cpu_rows)

    out = {
        "metric": "block-causal attn TFLOP/s (% bf16 MFMA peak) + ms/wave round, 832x480, 7 chunks",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "round": t_meas,
            "policy": wi.POLICY_NAMES[policy],
            "chunks": w.B, "levels": w.K, "chunk_tokens": w.chunk_len, "cond_tokens": w.cond_len,
            "heads": w.heads, "head_dim": w.head_dim, "history_cap": w.history_cap,
            "nodes_in_round": len(nodes), "query_rows": rows, "query_rows_per_node": qlen,
            "splitkv_splits": splits if decode else None,
            "tail_cut_items": None if decode else tail[0],
            "tail_cut_splits": None if decode else tail[1],
            "algorithmic_tflop": round(flops / 1e12, 4),
        },
        "attn_ms": round(attn_avg, 4),
        "attn_ms_median": round(float(np.median(attn_ms)), 4),
        "attn_ms_p10": round(float(np.percentile(attn_ms, 10)), 4),
        "attn_ms_p90": round(float(np.percentile(attn_ms, 90)), 4),
        "kv_write_ms": round(float(kvw_ms.mean()), 4),
        "round_ms": round(attn_avg + float(kvw_ms.mean()), 4),
        "pct_bf16_peak": round(100 * achieved / PEAK_BF16_TFLOPS, 2),
        "kv_write_gbps": round(kvw_bytes / (kvw_ms.mean() * 1e-3) / 1e9, 1),
        "plan_ms": round(plan_ms, 3),
        "roofline": ({
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profile(key),
        } if not decode else {
            "bound": "hbm",
            "achieved": round(attn_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic_from_profile(key),
        }),
        "attn_compulsory_mb": round(attn_bytes / 1e6, 2),
        "attn_gbps": round(attn_gbps, 1),
        "cpu_baseline": cpu_res,
    }
    if copy_ms is not None:
        out["copy_1gib_ms"] = round(copy_ms, 4)
    del cache, q, o, lse, k_src, v_src, workspace
    torch.cuda.empty_cache()
    return out


def chain_bench(args, device):
    """Whole rollouts of the toy denoiser chain at the Wan2.1-1.3B shape: per
    round and layer, qkv_project (K/V straight into the layer's cache, Q out)
    then wave_attn; chain_store after the last layer.  Every node's input is
    its chunk's previous output (seeded noise for the first update)."""
    import torch
    import block_causal_attention_wave_amd as wv
    import wave_inputs as wi
    key = args.workload if args.workload in (3, 4) else 3
    w = wi.WORKLOADS[key]
    layers = args.layers or w.layers
    D = w.heads * w.head_dim
    stream = torch.cuda.Stream()
    results = []
    for policy in ((wi.PROGRESSIVE,) if key == 3 else w.policies):
        plan = wv.wave_plan(B=w.B, K=w.K, policy=policy, sched=wv.WAVE, chunk_len=w.chunk_len,
                            history_cap=w.history_cap)
        desc = plan.upload(device)
        caches = [wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, plan.lpad(), device, fill=float("nan"))
                  for _ in range(layers)]
        weights = [wi.device_chain_weight(w.key, l, D, device) for l in range(layers)]
        state = torch.stack([wi.device_chain_noise(w.key, c, w.chunk_len, D, device) for c in range(w.B)])
        max_rows = int(plan.round_q_rows.max())
        q = torch.empty((max_rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=device)
        o = [torch.empty((max_rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=device) for _ in range(2)]
        proj_ws = torch.empty(max_rows * 4 + 256, dtype=torch.uint8, device=device)
        # per-head sums of squares of each layer's O: the next layer's RMS
        sq = [torch.empty((max_rows, w.heads), dtype=torch.float32, device=device) for _ in range(2)]
        fused = not args.no_fused_rms
        attn_bytes = max(wv.attn_workspace(plan, t, w.heads, w.head_dim)[0] for t in range(plan.num_rounds))
        attn_ws = torch.empty(max(attn_bytes, 1), dtype=torch.uint8, device=device)
        proj_ms = attn_ms = store_ms = 0.0
        proj_flops = attn_flops = 0.0
        round_ms = np.zeros(plan.num_rounds)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for t in range(plan.num_rounds):
                rows = int(plan.round_q_rows[t])
                attn_flops += algorithmic_flops(plan, t, w.heads, w.head_dim) * layers
                proj_flops += 2.0 * rows * D * 3 * D * layers
                x, layout, x_sq = state, wv.X_CHUNK, None
                for layer in range(layers):
                    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                    ev[0].record(stream)
                    wv.qkv_project(plan, desc, t, caches[layer], x, weights[layer], q=q[:rows], x_layout=layout,
                                   workspace=proj_ws, stream=stream, row_sq=x_sq)
                    ev[1].record(stream)
                    ob = o[layer & 1][:rows]
                    o_sq = sq[layer & 1] if fused else None
                    wv.wave_attn(plan, desc, t, caches[layer], q[:rows], w.scale, o=ob, want_lse=False,
                                 stream=stream, workspace=attn_ws, row_sq=o_sq)
                    ev[2].record(stream)
                    ev[2].synchronize()
                    proj_ms += ev[0].elapsed_time(ev[1])
                    attn_ms += ev[1].elapsed_time(ev[2])
                    round_ms[t] += ev[0].elapsed_time(ev[2])
                    x, layout, x_sq = ob.view(rows, D), wv.X_ROUND, o_sq
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                wv.chain_store(plan, desc, t, o[(layers - 1) & 1][:rows], state, stream=stream)
                e1.record(stream)
                e1.synchronize()
                store_ms += e0.elapsed_time(e1)
                round_ms[t] += e0.elapsed_time(e1)
        finite = bool(torch.isfinite(state.float()).all())
        del caches, weights
        torch.cuda.empty_cache()
        total = float(round_ms.sum())
        calls = plan.num_rounds * layers
        res = {
            "policy": wi.POLICY_NAMES[policy], "layers": layers, "rounds": plan.num_rounds,
            "rms_from_attention": fused,
            "total_ms": round(total, 3), "ms_per_round": round(total / plan.num_rounds, 3),
            "ms_per_chunk": round(total / w.B, 3),
            "attention_tflops": round(attn_flops / (attn_ms * 1e-3) / 1e12, 1),
            "projection_tflops": round(proj_flops / (proj_ms * 1e-3) / 1e12, 1),
            "projection_ms_per_call": round(proj_ms / calls, 4),
            "attention_ms_per_call": round(attn_ms / calls, 4),
            "chain_store_ms_per_round": round(store_ms / plan.num_rounds, 4),
            "projection_share": round(proj_ms / total, 4),
            "finite": finite,
        }
        eprint(f"[chain] {w.name} {res['policy']}: {plan.num_rounds} rounds x {layers} layers, {total:.1f} ms "
               f"total, {res['ms_per_round']:.2f} ms/round, {res['ms_per_chunk']:.2f} ms/chunk; attention "
               f"{res['attention_tflops']:.0f} TFLOP/s, projection {res['projection_tflops']:.0f} TFLOP/s "
               f"({res['projection_ms_per_call']:.3f} ms/call, {100 * res['projection_share']:.1f}% of the time)")
        results.append(res)
    print(json.dumps({"metric": "toy-chain rollout ms per round / per chunk; attention and projection TFLOP/s",
                      "workload": w.name + "-toy-chain", "unit": "ms", "n_gpus": 1, "dtype": "bf16",
                      "data": "synthetic", "timing": "sum of per-(round, layer) qkv_project + wave_attn and "
                      "per-round chain_store event times", "results": results}), flush=True)


def proj_bench(args, device):
    """qkv_project (RMS scaling, Q out, K/V^T into the node's cache slot) and
    the plain product x @ W^T of the same shape through torch.matmul, on the
    same GPU in one run: one round per distinct node count of the Wan2.1-1.3B
    progressive plan, alternating the three, timed with events.  qkv_project
    runs twice: with 1/rms taken from x's rows (a separate row-scale launch
    first) and with it formed from per-(row, head) sums of squares handed in,
    as the chain hands over the ones its attention epilogue wrote (here they
    are computed from x outside the timed calls)."""
    import torch
    import block_causal_attention_wave_amd as wv
    import wave_inputs as wi
    w = wi.WORKLOADS[3]
    D = w.heads * w.head_dim
    plan = wv.wave_plan(B=w.B, K=w.K, policy=wi.PROGRESSIVE, sched=wv.WAVE, chunk_len=w.chunk_len,
                        history_cap=w.history_cap)
    desc = plan.upload(device)
    cache = wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, plan.lpad(), device, fill=0.0)
    weight = wi.device_chain_weight(w.key, 0, D, device)
    weight_t = weight.t().contiguous()  # [D, 3D] for the plain product
    by_count = {}
    for t in range(plan.num_rounds):
        by_count.setdefault(len(plan.round_nodes(t)), t)
    max_rows = int(plan.round_q_rows.max())
    x_all = wi.device_normal_bf16(wi.chain_noise_seed(w.key, 0), (max_rows, D), 1.0, device)
    q = torch.empty((max_rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=device)
    y = torch.empty((max_rows, 3 * D), dtype=torch.bfloat16, device=device)
    ws = torch.empty(max_rows * 4 + 256, dtype=torch.uint8, device=device)
    stream = torch.cuda.Stream()
    reps, warm = max(args.steps // 5, 5), 3
    results = []
    with torch.cuda.stream(stream):
        for count, t in sorted(by_count.items()):
            rows = int(plan.round_q_rows[t])
            x = x_all[:rows]
            flops = 2.0 * rows * D * 3 * D
            sq = x.float().reshape(rows, w.heads, w.head_dim).square().sum(-1).contiguous()

            def proj():
                wv.qkv_project(plan, desc, t, cache, x, weight, q=q[:rows], x_layout=wv.X_ROUND, workspace=ws,
                               stream=stream)

            def proj_sq():
                wv.qkv_project(plan, desc, t, cache, x, weight, q=q[:rows], x_layout=wv.X_ROUND, workspace=ws,
                               stream=stream, row_sq=sq)

            def plain():
                torch.matmul(x, weight_t, out=y[:rows])

            fns = (("qkv_project", proj), ("qkv_project_rms_from_sq", proj_sq), ("torch.matmul", plain))
            for _ in range(warm):
                for _name, fn in fns:
                    fn()
            times = {name: [] for name, _fn in fns}
            for r in range(reps):
                for name, fn in fns:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    e1.synchronize()
                    times[name].append(e0.elapsed_time(e1))
            res = {"nodes": count, "round": t, "rows": rows, "gflop": round(flops / 1e9, 2)}
            for name, ts in times.items():
                med = float(np.median(ts))
                res[name + "_ms"] = round(med, 4)
                res[name + "_tflops"] = round(flops / (med * 1e-3) / 1e12, 1)
            eprint(f"[proj] {count} nodes, {rows} rows: qkv_project {res['qkv_project_ms']:.4f} ms = "
                   f"{res['qkv_project_tflops']:.0f} TFLOP/s; with the sums of squares handed in "
                   f"{res['qkv_project_rms_from_sq_ms']:.4f} ms = {res['qkv_project_rms_from_sq_tflops']:.0f} "
                   f"TFLOP/s; torch.matmul {res['torch.matmul_ms']:.4f} ms = "
                   f"{res['torch.matmul_tflops']:.0f} TFLOP/s")
            results.append(res)
    print(json.dumps({"metric": "qkv_project TFLOP/s against the plain product of the same shape",
                      "workload": w.name + "-qkv-projection", "unit": "TFLOP/s", "n_gpus": 1, "dtype": "bf16",
                      "data": "synthetic", "timing": "median of per-call event times, the three alternating",
                      "results": results}), flush=True)


def tiny_bench(args, device):
    """The tiny workload (B=4, K=2, 128-token chunks, 2 heads of 64, fp32 inputs)
    as a whole: every round's kv_write + wave_attn on the GPU, timed per
    rollout, beside the full fp64 CPU oracle of the same rollout (every node,
    row and head), with the parity of the last GPU rollout against it.  Parity,
    not throughput, is what this size shows."""
    import torch
    import block_causal_attention_wave_amd as wv
    import wave_inputs as wi
    from oracle import plan as op
    from oracle.attention import round_to_bf16
    from oracle.rollout import rollout
    w = wi.WORKLOADS[1]
    policy = w.policies[0]
    plan = wv.wave_plan(B=w.B, K=w.K, policy=policy, sched=wv.WAVE, chunk_len=w.chunk_len, cond_len=w.cond_len)
    desc = plan.upload(device)
    cache = wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, plan.lpad(), device, fill=float("nan"))
    host = {}

    def host_in(c, lv, which):
        if (c, lv, which) not in host:
            host[(c, lv, which)] = wi.host_tensor(w, 0, c, lv, which, policy)
        return host[(c, lv, which)]

    rounds = []
    for t in range(plan.num_rounds):
        ws = plan.round_writes(t).tolist()
        nodes = plan.round_nodes(t).tolist()
        k = torch.from_numpy(np.concatenate([host_in(c, lv, "k") for (c, lv, _, _) in ws])).to(device)
        v = torch.from_numpy(np.concatenate([host_in(c, lv, "v") for (c, lv, _, _) in ws])).to(device)
        q = torch.from_numpy(np.concatenate([host_in(n[0], n[1], "q") for n in nodes])).to(device)
        rows = int(plan.round_q_rows[t])
        o = torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=device)
        lse = torch.empty((w.heads, rows), dtype=torch.float32, device=device)
        rounds.append((t, k, v, q, o, lse, nodes))
    stream = torch.cuda.Stream()
    times = []
    with torch.cuda.stream(stream):
        for it in range(args.warmup + args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for (t, k, v, q, o, lse, _) in rounds:
                wv.kv_write(plan, desc, t, cache, k, v, stream=stream)
                wv.wave_attn(plan, desc, t, cache, q, w.scale, o=o, lse=lse, stream=stream)
            e1.record(stream)
            e1.synchronize()
            if it >= args.warmup:
                times.append(e0.elapsed_time(e1))
    gpu_ms = float(np.median(times))
    got = {}
    for (t, k, v, q, o, lse, nodes) in rounds:
        o_h, l_h = o.float().cpu().numpy(), lse.cpu().numpy()
        for n in nodes:
            got[(n[0], n[1])] = (o_h[n[4]:n[4] + n[5]], l_h[:, n[4]:n[4] + n[5]])
    # The full oracle on the values the kernels consume (fp32 rounded to bf16, widened to fp64).
    p = op.Params(w.B, w.K, policy, op.SERIAL, w.history_cap, w.chunk_len, w.cond_len, 0)
    oplan = op.oracle_plan(p)
    q64 = {key[:2]: round_to_bf16(x).astype(np.float64) for key, x in host.items() if key[2] == "q"}
    kv64 = {key[:2]: (round_to_bf16(host[key[:2] + ("k",)]).astype(np.float64),
                      round_to_bf16(host[key[:2] + ("v",)]).astype(np.float64))
            for key in host if key[2] == "k"}
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", affinity))
    t0 = time.perf_counter()
    ref = rollout(p, oplan, lambda c, lv: q64[(c, lv)], lambda c, lv: kv64[(c, lv)], w.scale)
    cpu_ms = (time.perf_counter() - t0) * 1e3
    assert set(ref) == set(got)
    err_o = max(float(np.abs(got[key][0] - ref[key][0]).max()) for key in ref)
    err_l = max(float(np.abs(got[key][1] - ref[key][1]).max()) for key in ref)
    flops = sum(algorithmic_flops(plan, t, w.heads, w.head_dim) for t in range(plan.num_rounds))
    eprint(f"[bench] {w.name}: whole rollout ({plan.num_rounds} rounds, {len(ref)} nodes) {gpu_ms:.3f} ms on the "
           f"GPU, {cpu_ms:.1f} ms for the full fp64 oracle ({threads} threads); max |dO| {err_o:.2e}, "
           f"max |dLSE| {err_l:.2e}")
    print(json.dumps({
        "metric": "tiny workload: whole-rollout time, GPU beside the full CPU oracle (parity size)",
        "value": round(gpu_ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "rounds": plan.num_rounds, "nodes": len(ref), "heads": w.heads,
                   "head_dim": w.head_dim, "chunk_tokens": w.chunk_len, "src_dtype": "fp32",
                   "algorithmic_gflop": round(flops / 1e9, 4)},
        "parity": {"max_abs_o": err_o, "max_abs_lse": err_l},
        "cpu_baseline": {"value": round(cpu_ms, 2), "unit": "ms", "cores": int(threads), "kind": "oracle",
                         "affinity_cpus": affinity,
                         "sample": "the whole rollout: every node, query row and head, fp64 dense masks"},
    }), flush=True)


def rollout_bench(args, device):
    """Whole pipelined rollouts through the round driver: one wave_round call per round
    (kv_write then wave_attn for every layer), timed per round, synchronised once."""
    import torch
    import block_causal_attention_wave_amd as wv
    import wave_inputs as wi
    key = args.workload if args.workload in (3, 4) else 3
    w = wi.WORKLOADS[key]
    layers = args.layers or w.layers
    stream = torch.cuda.Stream()
    results = []
    for policy in w.policies:
        plan = wv.wave_plan(B=w.B, K=w.K, policy=policy, sched=wv.WAVE, chunk_len=w.chunk_len,
                            cond_len=w.cond_len, history_cap=w.history_cap)
        desc = plan.upload(device)
        caches = [wv.KVCache(plan.num_phys_slots, w.heads, w.head_dim, plan.lpad(), device, fill=float("nan"))
                  for _ in range(layers)]
        ws_bytes = max(wv.attn_workspace(plan, t, w.heads, w.head_dim)[0] for t in range(plan.num_rounds))
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
        flops = 0.0
        events, finite = [], []
        with torch.cuda.stream(stream):
            stream.wait_stream(torch.cuda.default_stream(device))
            for t in range(plan.num_rounds):
                rows = int(plan.round_q_rows[t])
                flops += algorithmic_flops(plan, t, w.heads, w.head_dim) * layers
                ws = plan.round_writes(t).tolist()
                nodes = plan.round_nodes(t).tolist()
                # the round's inputs for every layer, generated before its timed region
                ks = [torch.cat([wi.device_tensor(w, l, c, lv, "k", device, policy) for (c, lv, _, _) in ws])
                      for l in range(layers)]
                vs = [torch.cat([wi.device_tensor(w, l, c, lv, "v", device, policy) for (c, lv, _, _) in ws])
                      for l in range(layers)]
                qs = [torch.cat([wi.device_tensor(w, l, n[0], n[1], "q", device, policy) for n in nodes])
                      for l in range(layers)]
                os_ = [torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=device)
                       for _ in range(layers)]
                lses = [torch.empty((w.heads, rows), dtype=torch.float32, device=device) for _ in range(layers)]
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                wv.wave_round(plan, desc, t, caches, ks, vs, qs, w.scale, os=os_, lses=lses, stream=stream,
                              workspace=workspace)
                e1.record(stream)
                events.append((e0, e1))
                finite.append(torch.stack([torch.isfinite(x).all() for x in lses]).all())
                del ks, vs, qs, os_, lses
        stream.synchronize()
        round_ms = np.array([e0.elapsed_time(e1) for e0, e1 in events])
        finite = bool(torch.stack(finite).all())
        del caches
        torch.cuda.empty_cache()
        total = float(round_ms.sum())
        # steady rounds: every level in flight (and, with a history cap, a full window)
        first = w.K + (w.history_cap if w.history_cap >= 0 else 0)
        steady = round_ms[first:w.B] if w.B > first else round_ms
        res = {
            "policy": wi.POLICY_NAMES[policy], "layers": layers, "rounds": plan.num_rounds,
            "total_ms": round(total, 3), "ms_per_round": round(total / plan.num_rounds, 3),
            "ms_per_chunk": round(total / w.B, 3), "tflop": round(flops / 1e12, 2),
            "tflops": round(flops / (float(round_ms.sum()) * 1e-3) / 1e12, 1),
            "steady_round_ms": {"median": round(float(np.median(steady)), 3),
                                "p10": round(float(np.percentile(steady, 10)), 3),
                                "p90": round(float(np.percentile(steady, 90)), 3)},
            "finite": finite,
        }
        eprint(f"[rollout] {w.name} {res['policy']}: {plan.num_rounds} rounds x {layers} layers, "
               f"{total:.1f} ms total, {res['ms_per_round']:.2f} ms/round, {res['ms_per_chunk']:.2f} ms/chunk, "
               f"{res['tflops']:.0f} TFLOP/s (attention FLOPs over round time, kv_write included), "
               f"steady round median {res['steady_round_ms']['median']} ms")
        results.append(res)
    print(json.dumps({"metric": "wave rollout ms per round / per chunk + attention TFLOP/s", "workload": w.name,
                      "unit": "ms", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
                      "timing": "sum of per-round wave_round event times (kv_write + wave_attn of every layer, "
                                "one call per round, no host sync inside the rollout)",
                      "results": results}), flush=True)


def cpu_baseline(w, plan, t_meas, nodes, policy, layer, device, rows_per_node):
    """The CPU oracle on a bounded sample of the same round: `rows_per_node`
    query rows of every node, all heads, fp64 with explicit dense masks."""
    import torch
    import wave_inputs as wi
    from oracle import plan as op
    from oracle.rollout import rollout
    # The oracle's dense products run on numpy's BLAS thread pool, which takes
    # the process's CPU share (OMP_NUM_THREADS where it is set, else every CPU
    # the process may run on); `cores` is that pool's size, the threads used.
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", affinity))

    qlen = w.query_len or w.chunk_len
    p = op.Params(w.B, w.K, policy, op.SERIAL, w.history_cap, w.chunk_len, w.cond_len, w.query_len)
    oplan = op.oracle_plan(p)
    want = {(n[0], n[1]) for n in nodes}
    rows = sample_rows(qlen, rows_per_node)
    # Every slot the serial rollout writes until it reaches the wanted nodes:
    # fetched from the seeded generator before the clock starts.
    need = set()
    done = set()
    for t in range(oplan["num_rounds"]):
        for nd in oplan["nodes"][oplan["round_node_begin"][t]:oplan["round_node_begin"][t + 1]]:
            for wr in oplan["writes"][nd[8]:nd[8] + nd[9]]:
                need.add((wr[0], wr[1]))
            if (nd[0], nd[1]) in want:
                done.add((nd[0], nd[1]))
        if done == want:
            break
    kv = {}
    for (c, lv) in need:
        k = wi.device_tensor(w, layer, c, lv, "k", device, policy).float().cpu().numpy().astype(np.float64)
        v = wi.device_tensor(w, layer, c, lv, "v", device, policy).float().cpu().numpy().astype(np.float64)
        kv[(c, lv)] = (k, v)
    qs = {(c, lv): wi.device_tensor(w, layer, c, lv, "q", device, policy)[-qlen:].float().cpu().numpy()
          .astype(np.float64) for (c, lv) in want}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = rollout(p, oplan, lambda c, lv: qs[(c, lv)], lambda c, lv: kv[(c, lv)], w.scale,
                  rows=lambda c, lv: rows, want=want)
    secs = time.perf_counter() - t0
    assert set(out) == want
    flops = algorithmic_flops(plan, t_meas, w.heads, w.head_dim, rows_per_node=len(rows))
    eprint(f"[bench] cpu oracle: {len(rows)} rows x {len(nodes)} nodes x {w.heads} heads in {secs:.1f} s "
           f"({threads} threads) = {flops / secs / 1e9:.2f} GFLOP/s")
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "affinity_cpus": affinity,
        "sample": f"{len(rows)} query rows of each of the {len(nodes)} nodes of round {t_meas}, "
                  f"all {w.heads} heads, fp64 dense-mask attention over every live slot; "
                  f"{secs:.1f} s wall; full-round estimate {secs * qlen / len(rows):.0f} s",
    }


if __name__ == "__main__":
    main()
