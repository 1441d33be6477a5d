"""The allocation-free split-KV entry point (wave_attn_splitkv_noalloc)
against the workspace entry point (wave_attn_splitkv), both called through
the C ABI: two calls of the allocation-free one in a row, the second on a
smaller input (its scratch still holding the first call's partials), each
bitwise equal to the workspace entry point with the same split count."""
import ctypes as C

import numpy as np
import pytest

import block_causal_attention_wave_amd as wv
from block_causal_attention_wave_amd import _lib
from gpu_common import log
import wave_inputs as wi

pytestmark = pytest.mark.gpu

# (B, K, policy, chunk_len, cond_len, query_len, heads, head_dim, splits)
CASES = [
    # Wan-Streamer-shaped audio decode (640x368 chunks of 2760 video + 64 audio
    # tokens, 512-token conditioning slices, 40 heads), library's split count
    (6, 2, wi.SAME_LEVEL, 2824, 512, 64, 40, 128, 0),
    # a smaller round: fewer rows, heads and keys, head_dim 64, 5 splits
    (3, 2, wi.PROGRESSIVE, 700, 0, 16, 8, 64, 5),
]


def _setup(device, case, key):
    import torch
    B, K, pol, L, cond, qlen, heads, hd, splits = case
    plan = wv.wave_plan(B=B, K=K, policy=pol, sched=wv.WAVE, chunk_len=L, cond_len=cond, query_len=qlen)
    desc = plan.upload(device)
    cache = wv.KVCache(plan.num_phys_slots, heads, hd, plan.lpad(), device, fill=float("nan"))
    last = plan.num_rounds - 1

    def t_(c, lv, which, n):
        return wi.device_normal_bf16(wi.tensor_seed(key, 0, c, lv, which, pol), (n, heads, hd), 1.0, device)

    for t in range(last + 1):
        ws = plan.round_writes(t).tolist()
        k = torch.cat([t_(c, lv, "k", ln) for (c, lv, _p, ln) in ws])
        v = torch.cat([t_(c, lv, "v", ln) for (c, lv, _p, ln) in ws])
        wv.kv_write(plan, desc, t, cache, k, v)
    q = torch.cat([t_(n[0], n[1], "q", qlen) for n in plan.round_nodes(last).tolist()])
    return dict(plan=plan, desc=desc, cache=cache, round=last, q=q, scale=float(hd) ** -0.5, splits=splits)


def _call(lib, s, workspace=None):
    import torch
    plan, cache, q = s["plan"], s["cache"], s["q"]
    rows = int(plan.round_q_rows[s["round"]])
    o = torch.empty((rows, cache.heads, cache.head_dim), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((cache.heads, rows), dtype=torch.float32, device=q.device)
    common = (plan.handle, C.c_void_p(s["desc"].data_ptr()), s["round"], C.byref(cache.c),
              C.c_void_p(q.data_ptr()), _lib.WAVE_DTYPE_BF16, q.stride(0), C.c_void_p(o.data_ptr()),
              C.c_void_p(lse.data_ptr()), s["scale"], s["splits"])
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if workspace is None:
        rc = lib.wave_attn_splitkv_noalloc(*common, stream)
    else:
        rc = lib.wave_attn_splitkv(*common, C.c_void_p(workspace.data_ptr()), workspace.numel(), stream)
    _lib.check(rc)
    return o, lse


def test_noalloc_splitkv_equals_workspace_entry_point(gpu_device):
    import torch
    lib = _lib.load()
    setups = []
    for i, case in enumerate(CASES):
        log(f"no-alloc split-KV case {i}: {case}")
        setups.append(_setup(gpu_device, case, 900 + i))
    torch.cuda.synchronize()
    for s in setups:
        nbytes, used = wv.splitkv_workspace_bytes(s["plan"], s["round"], s["cache"].heads, s["cache"].head_dim,
                                                  s["splits"])
        assert used > 1 and 0 < nbytes <= _lib.WAVE_NOALLOC_SCRATCH_BYTES
        s["nbytes"] = nbytes
    # Two calls in a row, the second on the smaller input.
    got = [_call(lib, s) for s in setups]
    torch.cuda.synchronize()
    for i, (s, (o, lse)) in enumerate(zip(setups, got)):
        ws = torch.empty(s["nbytes"], dtype=torch.uint8, device=gpu_device)
        o_ref, lse_ref = _call(lib, s, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all(), f"case {i}"
        assert torch.equal(o, o_ref), f"case {i}: O differs from wave_attn_splitkv"
        assert torch.equal(lse, lse_ref), f"case {i}: LSE differs from wave_attn_splitkv"
        log(f"  case {i}: {o.shape[0]} rows x {o.shape[1]} heads bitwise equal ({s['nbytes']} bytes of scratch)")
    # A split count whose partials exceed the scratch is refused before any launch.
    big = dict(setups[0], splits=64)
    nbytes, _ = wv.splitkv_workspace_bytes(big["plan"], big["round"], big["cache"].heads,
                                           big["cache"].head_dim, 64)
    assert nbytes > _lib.WAVE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(wv.WaveError) as e:
        _call(lib, big)
    assert e.value.code == _lib.WAVE_ERR_CAPACITY
