"""Chunk-wise block-causal wave attention on AMD MI355X (gfx950).

Thin Python binding of ``include/wave.h`` (libwave.so): argument marshalling
only.  PyTorch supplies device memory and streams; every step of the path
(planning, K/V cache writes, attention) runs in the native library.  There is
no fallback: if libwave.so is missing, importing the binding functions raises.

    plan  = wave_plan(B=7, K=4, policy=PROGRESSIVE, sched=WAVE, chunk_len=4680)
    desc  = plan.upload(device)
    cache = KVCache(plan.num_phys_slots, heads=12, head_dim=128,
                    lpad=plan.lpad(), device=device)
    for t in range(plan.num_rounds):
        kv_write(plan, desc, t, cache, k_fresh[t], v_fresh[t])
        o, lse = wave_attn(plan, desc, t, cache, q[t], scale=128 ** -0.5)
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib
from ._lib import (WAVE_CLEAN, WAVE_DTYPE_BF16, WAVE_DTYPE_FP32, WAVE_KEY_TILE, WAVE_LEVEL_COND,
                   WAVE_NODE_REFRESH, WAVE_NODE_UPDATE, WAVE_PROGRESSIVE, WAVE_Q_TILE,
                   WAVE_SAME_LEVEL, WAVE_SCHED_SERIAL, WAVE_SCHED_WAVE, WaveError)

CLEAN, SAME_LEVEL, PROGRESSIVE = WAVE_CLEAN, WAVE_SAME_LEVEL, WAVE_PROGRESSIVE
SERIAL, WAVE = WAVE_SCHED_SERIAL, WAVE_SCHED_WAVE

__all__ = ["Plan", "KVCache", "wave_plan", "kv_write", "wave_attn", "wave_round", "wave_attn_splitkv",
           "wave_attn_splitkv_noalloc",
           "attn_workspace", "splitkv_workspace_bytes", "qkv_project", "chain_store", "WaveError",
           "CLEAN", "SAME_LEVEL", "PROGRESSIVE", "SERIAL", "WAVE", "WAVE_LEVEL_COND",
           "WAVE_Q_TILE", "WAVE_KEY_TILE", "WAVE_NODE_UPDATE", "WAVE_NODE_REFRESH"]


def _arr(ptr, n, cols):
    if n == 0:
        return np.zeros((0, cols) if cols else (0,), dtype=np.int32)
    buf = C.cast(ptr, C.POINTER(C.c_int32 * (n * (cols or 1)))).contents
    a = np.frombuffer(buf, dtype=np.int32).copy()
    return a.reshape(n, cols) if cols else a


class Plan:
    """A host plan (``wave_plan``) with numpy copies of its view arrays.

    nodes : [N, 10] chunk, level, kind, round, q_offset, q_len, ctx_begin,
            ctx_count, write_begin, write_count
    ctx, writes : [*, 4] chunk, level, phys_slot, len
    work : [*, 4] node, q_start, q_rows, keys
    """

    def __init__(self, B, K, policy, sched, chunk_len, history_cap=-1, cond_len=0, q_tile=0,
                 query_len=0):
        lib = _lib.load()
        self.params = dict(B=B, K=K, policy=policy, sched=sched, history_cap=history_cap,
                           chunk_len=chunk_len, cond_len=cond_len, q_tile=q_tile, query_len=query_len)
        p = _lib.PlanParams(B, K, policy, sched, history_cap, chunk_len, cond_len, q_tile, query_len)
        h = C.c_void_p()
        _lib.check(lib.wave_plan(C.byref(p), C.byref(h)))
        self._h = h
        v = _lib.PlanView()
        _lib.check(lib.wave_plan_view_get(h, C.byref(v)))
        self.num_rounds = v.num_rounds
        self.num_phys_slots = v.num_phys_slots
        self.max_slot_len = v.max_slot_len
        self.q_tile = v.q_tile
        self.round_node_begin = _arr(v.round_node_begin, v.num_rounds + 1, 0)
        self.round_write_begin = _arr(v.round_write_begin, v.num_rounds + 1, 0)
        self.round_work_begin = _arr(v.round_work_begin, v.num_rounds + 1, 0)
        self.round_q_rows = _arr(v.round_q_rows, v.num_rounds, 0)
        self.round_src_rows = _arr(v.round_src_rows, v.num_rounds, 0)
        self.nodes = _arr(v.nodes, v.num_nodes, 10)
        self.ctx = _arr(v.ctx, v.num_ctx, 4)
        self.writes = _arr(v.writes, v.num_writes, 4)
        self.work = _arr(v.work, v.num_work, 4)
        size = C.c_size_t()
        _lib.check(lib.wave_plan_desc_size(h, C.byref(size)))
        self._desc = np.zeros(size.value // 4, dtype=np.int32)
        _lib.check(lib.wave_plan_desc_pack(h, self._desc.ctypes.data_as(C.c_void_p), size.value))

    @property
    def handle(self):
        return self._h

    def desc(self) -> np.ndarray:
        return self._desc.copy()

    def upload(self, device):
        import torch
        return torch.from_numpy(self._desc.copy()).to(device)

    def lpad(self) -> int:
        return -(-self.max_slot_len // WAVE_KEY_TILE) * WAVE_KEY_TILE

    def round_nodes(self, t):
        return self.nodes[self.round_node_begin[t]:self.round_node_begin[t + 1]]

    def round_writes(self, t):
        return self.writes[self.round_write_begin[t]:self.round_write_begin[t + 1]]

    def node_ctx(self, n):
        return self.ctx[n[6]:n[6] + n[7]]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib.load().wave_plan_destroy(h)
            self._h = None


def wave_plan(**kw) -> Plan:
    return Plan(**kw)


class KVCache:
    """One layer's cache: K [slots][heads][lpad][d] and V^T [slots][heads][d][lpad], bf16."""

    def __init__(self, num_slots, heads, head_dim, lpad, device, fill=None):
        import torch
        self.k = torch.empty((num_slots, heads, lpad, head_dim), dtype=torch.bfloat16, device=device)
        self.vt = torch.empty((num_slots, heads, head_dim, lpad), dtype=torch.bfloat16, device=device)
        if fill is not None:
            self.k.fill_(fill)
            self.vt.fill_(fill)
        self.num_slots, self.heads, self.head_dim, self.lpad = num_slots, heads, head_dim, lpad
        self._c = _lib.KvCache(self.k.data_ptr(), self.vt.data_ptr(), num_slots, heads, head_dim, lpad)

    @property
    def c(self):
        return self._c


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return WAVE_DTYPE_BF16
    if t.dtype == torch.float32:
        return WAVE_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_rows(t, rows, heads, head_dim, what):
    if t.dim() != 3 or t.shape[0] != rows or t.shape[1] != heads or t.shape[2] != head_dim:
        raise ValueError(f"{what}: expected [{rows}, {heads}, {head_dim}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != head_dim:
        raise ValueError(f"{what}: heads and head_dim must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{what}: must be a device tensor")


def kv_write(plan: Plan, d_desc, round: int, cache: KVCache, k_src, v_src, stream=None) -> None:
    """Write round `round`'s fresh K/V ([rows, heads, d], bf16 or fp32) into `cache`."""
    rows = int(plan.round_src_rows[round]) if 0 <= round < plan.num_rounds else 0
    _check_rows(k_src, rows, cache.heads, cache.head_dim, "k_src")
    _check_rows(v_src, rows, cache.heads, cache.head_dim, "v_src")
    if k_src.dtype != v_src.dtype or k_src.stride(0) != v_src.stride(0):
        raise ValueError("k_src and v_src must share dtype and row stride")
    _lib.check(_lib.load().kv_write(plan.handle, C.c_void_p(d_desc.data_ptr()), round, C.byref(cache.c),
                                    C.c_void_p(k_src.data_ptr()), C.c_void_p(v_src.data_ptr()),
                                    _dtype_code(k_src), k_src.stride(0), _stream_ptr(stream)))


def _attn_outputs(plan, round, cache, q, o, lse, want_lse):
    import torch
    rows = int(plan.round_q_rows[round]) if 0 <= round < plan.num_rounds else 0
    _check_rows(q, rows, cache.heads, cache.head_dim, "q")
    if o is None:
        o = torch.empty((rows, cache.heads, cache.head_dim), dtype=torch.bfloat16, device=q.device)
    elif o.dtype != torch.bfloat16 or not o.is_contiguous() or tuple(o.shape) != (rows, cache.heads, cache.head_dim):
        raise ValueError("o must be a contiguous bf16 [rows, heads, d] tensor")
    if lse is None and want_lse:
        lse = torch.empty((cache.heads, rows), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                              or tuple(lse.shape) != (cache.heads, rows)):
        raise ValueError("lse must be a contiguous fp32 [heads, rows] tensor")
    return o, lse


def attn_workspace(plan: Plan, round: int, heads: int, head_dim: int, compute_units: int = 0):
    """(bytes, tail_items, tail_splits) of wave_attn's tail balancing for this round
    (compute_units 0 = the current device's)."""
    b = C.c_size_t()
    m = C.c_int32()
    s = C.c_int32()
    _lib.check(_lib.load().wave_attn_workspace(plan.handle, round, heads, head_dim, compute_units,
                                               C.byref(b), C.byref(m), C.byref(s)))
    return b.value, m.value, s.value


def wave_attn(plan: Plan, d_desc, round: int, cache: KVCache, q, scale: float, o=None, lse=None,
              want_lse=True, stream=None, balance=True, workspace=None, row_sq=None):
    """Attention of round `round`: q [rows, heads, d] (bf16 or fp32) -> (o bf16, lse fp32 [heads, rows]).

    balance: cut the round's trailing work items into key ranges when that
    shortens it (results then equal the unbalanced ones up to rounding); the
    workspace (uint8 tensor of attn_workspace() bytes) is allocated here when
    not given.  balance=False keeps each node's result bitwise independent of
    the schedule.

    row_sq: None, or an fp32 tensor [rows, heads] that receives each output
    row's per-head sum of squares of the bf16 O (wave_attn_chain), for the
    next layer's qkv_project(row_sq=...)."""
    import torch
    o, lse = _attn_outputs(plan, round, cache, q, o, lse, want_lse)
    ws_ptr, ws_bytes = 0, 0
    if balance:
        nbytes, _, _ = attn_workspace(plan, round, cache.heads, cache.head_dim)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    lse_ptr = C.c_void_p(lse.data_ptr() if lse is not None else 0)
    if row_sq is None:
        _lib.check(_lib.load().wave_attn(plan.handle, C.c_void_p(d_desc.data_ptr()), round, C.byref(cache.c),
                                         C.c_void_p(q.data_ptr()), _dtype_code(q), q.stride(0),
                                         C.c_void_p(o.data_ptr()), lse_ptr, float(scale), C.c_void_p(ws_ptr),
                                         ws_bytes, _stream_ptr(stream)))
    else:
        if (row_sq.dtype != torch.float32 or not row_sq.is_contiguous()
                or row_sq.numel() < int(plan.round_q_rows[round]) * cache.heads):
            raise ValueError("row_sq must be a contiguous float32 tensor of at least rows * heads elements")
        _lib.check(_lib.load().wave_attn_chain(plan.handle, C.c_void_p(d_desc.data_ptr()), round,
                                               C.byref(cache.c), C.c_void_p(q.data_ptr()), _dtype_code(q),
                                               q.stride(0), C.c_void_p(o.data_ptr()), lse_ptr, float(scale),
                                               C.c_void_p(row_sq.data_ptr()), C.c_void_p(ws_ptr), ws_bytes,
                                               _stream_ptr(stream)))
    return o, lse


def wave_round(plan: Plan, d_desc, round: int, caches, k_srcs, v_srcs, qs, scale: float, os=None, lses=None,
               want_lse=True, stream=None, balance=True, workspace=None):
    """One round of every layer in one call: for each layer, kv_write of its
    fresh K/V into caches[l], then wave_attn of qs[l], all enqueued on one
    stream with no host synchronisation.  k_srcs / v_srcs share a dtype and row
    stride, as do the qs.  Returns (os, lses), one entry per layer; the layers
    share one tail-balancing workspace (allocated here when not given)."""
    import torch
    n = len(caches)
    if n < 1 or not (len(k_srcs) == len(v_srcs) == len(qs) == n):
        raise ValueError("caches, k_srcs, v_srcs and qs need one entry per layer")
    if os is not None and len(os) != n or lses is not None and len(lses) != n:
        raise ValueError("os and lses need one entry per layer")
    rows = int(plan.round_src_rows[round]) if 0 <= round < plan.num_rounds else 0
    outs_o, outs_l = [], []
    for l in range(n):
        _check_rows(k_srcs[l], rows, caches[l].heads, caches[l].head_dim, f"k_srcs[{l}]")
        _check_rows(v_srcs[l], rows, caches[l].heads, caches[l].head_dim, f"v_srcs[{l}]")
        o, lse = _attn_outputs(plan, round, caches[l], qs[l], None if os is None else os[l],
                               None if lses is None else lses[l], want_lse)
        outs_o.append(o)
        outs_l.append(lse)
    for t in list(k_srcs) + list(v_srcs):
        if t.dtype != k_srcs[0].dtype or t.stride(0) != k_srcs[0].stride(0):
            raise ValueError("k_srcs and v_srcs must share one dtype and row stride")
    for t in qs:
        if t.dtype != qs[0].dtype or t.stride(0) != qs[0].stride(0):
            raise ValueError("qs must share one dtype and row stride")
    ws_ptr, ws_bytes = 0, 0
    if balance:
        nbytes = max(attn_workspace(plan, round, c.heads, c.head_dim)[0] for c in caches)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=qs[0].device)
        if workspace is not None:
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    cache_arr = (_lib.KvCache * n)(*[c.c for c in caches])

    def ptrs(ts):
        return (C.c_void_p * n)(*[t.data_ptr() if t is not None else 0 for t in ts])

    _lib.check(_lib.load().wave_round(plan.handle, C.c_void_p(d_desc.data_ptr()), round, n, cache_arr,
                                      ptrs(k_srcs), ptrs(v_srcs), _dtype_code(k_srcs[0]), k_srcs[0].stride(0),
                                      ptrs(qs), _dtype_code(qs[0]), qs[0].stride(0), ptrs(outs_o),
                                      ptrs(outs_l) if want_lse or lses is not None else None, float(scale),
                                      C.c_void_p(ws_ptr), ws_bytes, _stream_ptr(stream)))
    return outs_o, outs_l


def splitkv_workspace_bytes(plan: Plan, round: int, heads: int, head_dim: int, num_splits: int = 0):
    """(bytes, splits) of the split-KV workspace for this round (num_splits 0 = library's choice)."""
    b = C.c_size_t()
    s = C.c_int32()
    _lib.check(_lib.load().wave_attn_splitkv_workspace(plan.handle, round, heads, head_dim, num_splits,
                                                       C.byref(b), C.byref(s)))
    return b.value, s.value


def wave_attn_splitkv(plan: Plan, d_desc, round: int, cache: KVCache, q, scale: float, num_splits: int = 0,
                      workspace=None, o=None, lse=None, want_lse=True, stream=None):
    """Split-KV attention of round `round` (short queries, long contexts); same results as wave_attn."""
    import torch
    o, lse = _attn_outputs(plan, round, cache, q, o, lse, want_lse)
    nbytes, splits = splitkv_workspace_bytes(plan, round, cache.heads, cache.head_dim, num_splits)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _lib.check(_lib.load().wave_attn_splitkv(plan.handle, C.c_void_p(d_desc.data_ptr()), round,
                                             C.byref(cache.c), C.c_void_p(q.data_ptr()), _dtype_code(q),
                                             q.stride(0), C.c_void_p(o.data_ptr()),
                                             C.c_void_p(lse.data_ptr() if lse is not None else 0),
                                             float(scale), splits, C.c_void_p(workspace.data_ptr()),
                                             workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return o, lse


def wave_attn_splitkv_noalloc(plan: Plan, d_desc, round: int, cache: KVCache, q, scale: float,
                              num_splits: int = 0, o=None, lse=None, stream=None):
    """wave_attn_splitkv with its partial results in the library's per-device
    scratch array (no workspace, no device allocation by the library).  o and
    lse must be passed in for a call that allocates nothing at all; calls
    that overlap on one device race on the shared scratch."""
    o, lse = _attn_outputs(plan, round, cache, q, o, lse, lse is not None or o is None)
    _lib.check(_lib.load().wave_attn_splitkv_noalloc(plan.handle, C.c_void_p(d_desc.data_ptr()), round,
                                                     C.byref(cache.c), C.c_void_p(q.data_ptr()), _dtype_code(q),
                                                     q.stride(0), C.c_void_p(o.data_ptr()),
                                                     C.c_void_p(lse.data_ptr() if lse is not None else 0),
                                                     float(scale), int(num_splits), _stream_ptr(stream)))
    return o, lse


# --- toy denoiser chain: the steps on either side of the attention ---------------

X_ROUND, X_CHUNK = 0, 1


def qkv_project_workspace_bytes(plan: Plan, round: int) -> int:
    b = C.c_size_t()
    _lib.check(_lib.load().qkv_project_workspace(plan.handle, round, C.byref(b)))
    return b.value


def qkv_project(plan: Plan, d_desc, round: int, cache: KVCache, x, w, q=None, x_layout=X_ROUND,
                workspace=None, stream=None, row_sq=None):
    """QKV projection of every node of round `round` at one layer: K/V into the
    nodes' own slots of `cache`, Q returned ([rows, heads, head_dim] bf16).

    x: bf16 input rows, [round rows, D] (X_ROUND) or per-chunk state
    [B, chunk_len, D] (X_CHUNK); w: bf16 [3D, D].  row_sq: None, or the
    row_sq that wave_attn(row_sq=...) wrote with x as its o (X_ROUND only)."""
    import torch
    rows = int(plan.round_q_rows[round])
    if q is None:
        q = torch.empty((rows, cache.heads, cache.head_dim), dtype=torch.bfloat16, device=x.device)
    nbytes = qkv_project_workspace_bytes(plan, round)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
    _lib.check(_lib.load().qkv_project(plan.handle, C.c_void_p(d_desc.data_ptr()), round, C.byref(cache.c),
                                       C.c_void_p(x.data_ptr()), int(x_layout),
                                       C.c_void_p(row_sq.data_ptr() if row_sq is not None else 0),
                                       C.c_void_p(w.data_ptr()),
                                       C.c_void_p(q.data_ptr()), C.c_void_p(workspace.data_ptr()),
                                       workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return q


def chain_store(plan: Plan, d_desc, round: int, o, state, stream=None):
    """state[chunk of n] = o[rows of n] for every node n of round `round`
    (o: [round rows, ..., ] bf16 with D values per row; state: [B, chunk_len, D])."""
    model_dim = o[0].numel()
    _lib.check(_lib.load().chain_store(plan.handle, C.c_void_p(d_desc.data_ptr()), round, model_dim,
                                       C.c_void_p(o.data_ptr()), C.c_void_p(state.data_ptr()),
                                       _stream_ptr(stream)))
