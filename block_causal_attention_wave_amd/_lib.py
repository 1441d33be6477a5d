"""ctypes declarations of include/wave.h and the loader of libwave.so."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwave.so")

WAVE_OK = 0
WAVE_ERR_INVALID_ARG = -1
WAVE_ERR_CAPACITY = -2
WAVE_ERR_UNSUPPORTED = -3
WAVE_ERR_HIP = -4
WAVE_ERR_NOMEM = -5

WAVE_CLEAN, WAVE_SAME_LEVEL, WAVE_PROGRESSIVE = 0, 1, 2
WAVE_SCHED_SERIAL, WAVE_SCHED_WAVE = 0, 1
WAVE_NODE_UPDATE, WAVE_NODE_REFRESH = 0, 1
WAVE_DTYPE_BF16, WAVE_DTYPE_FP32 = 0, 1
WAVE_LEVEL_COND = -1
WAVE_Q_TILE = 256
WAVE_KEY_TILE = 64
WAVE_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ("wave_plan", "wave_plan_view_get", "wave_plan_desc_size", "wave_plan_desc_pack",
           "wave_plan_destroy", "kv_write", "wave_attn_workspace", "wave_attn", "wave_attn_splitkv_workspace",
           "wave_round", "wave_attn_splitkv", "wave_attn_splitkv_noalloc", "wave_attn_chain",
           "qkv_project_workspace", "qkv_project", "chain_store", "wave_last_error")


class PlanParams(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("B", "K", "policy", "sched", "history_cap", "chunk_len", "cond_len", "q_tile",
                 "query_len")]


class SlotRef(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("chunk", "level", "phys_slot", "len")]


class Node(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("chunk", "level", "kind", "round", "q_offset", "q_len",
                 "ctx_begin", "ctx_count", "write_begin", "write_count")]


class Work(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("node", "q_start", "q_rows", "keys")]


class PlanView(C.Structure):
    _fields_ = [
        ("num_rounds", C.c_int32), ("num_nodes", C.c_int32), ("num_ctx", C.c_int32),
        ("num_writes", C.c_int32), ("num_work", C.c_int32), ("num_phys_slots", C.c_int32),
        ("max_slot_len", C.c_int32), ("q_tile", C.c_int32),
        ("round_node_begin", C.POINTER(C.c_int32)),
        ("round_write_begin", C.POINTER(C.c_int32)),
        ("round_work_begin", C.POINTER(C.c_int32)),
        ("round_q_rows", C.POINTER(C.c_int32)),
        ("round_src_rows", C.POINTER(C.c_int32)),
        ("nodes", C.POINTER(Node)),
        ("ctx", C.POINTER(SlotRef)),
        ("writes", C.POINTER(SlotRef)),
        ("work", C.POINTER(Work)),
    ]


class KvCache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("vt", C.c_void_p), ("num_slots", C.c_int32),
                ("heads", C.c_int32), ("head_dim", C.c_int32), ("lpad", C.c_int32)]


_lib = None


def load() -> C.CDLL:
    """Load libwave.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_causal_attention_wave_amd.build`")
    lib = C.CDLL(LIB_PATH)
    lib.wave_plan.argtypes = [C.POINTER(PlanParams), C.POINTER(C.c_void_p)]
    lib.wave_plan.restype = C.c_int32
    lib.wave_plan_view_get.argtypes = [C.c_void_p, C.POINTER(PlanView)]
    lib.wave_plan_view_get.restype = C.c_int32
    lib.wave_plan_desc_size.argtypes = [C.c_void_p, C.POINTER(C.c_size_t)]
    lib.wave_plan_desc_size.restype = C.c_int32
    lib.wave_plan_desc_pack.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t]
    lib.wave_plan_desc_pack.restype = C.c_int32
    lib.wave_plan_destroy.argtypes = [C.c_void_p]
    lib.wave_plan_destroy.restype = None
    lib.kv_write.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(KvCache),
                             C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_void_p]
    lib.kv_write.restype = C.c_int32
    lib.wave_attn_workspace.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                        C.POINTER(C.c_size_t), C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    lib.wave_attn_workspace.restype = C.c_int32
    lib.wave_attn.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(KvCache),
                              C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p,
                              C.c_float, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.wave_attn.restype = C.c_int32
    P = C.POINTER(C.c_void_p)
    lib.wave_round.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.POINTER(KvCache), P, P,
                               C.c_int32, C.c_int64, P, C.c_int32, C.c_int64, P, P, C.c_float, C.c_void_p,
                               C.c_size_t, C.c_void_p]
    lib.wave_round.restype = C.c_int32
    lib.wave_attn_splitkv_workspace.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                                C.POINTER(C.c_size_t), C.POINTER(C.c_int32)]
    lib.wave_attn_splitkv_workspace.restype = C.c_int32
    lib.wave_attn_splitkv.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(KvCache),
                                      C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p,
                                      C.c_float, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.wave_attn_splitkv.restype = C.c_int32
    lib.wave_attn_splitkv_noalloc.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(KvCache),
                                              C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p,
                                              C.c_float, C.c_int32, C.c_void_p]
    lib.wave_attn_splitkv_noalloc.restype = C.c_int32
    lib.qkv_project_workspace.argtypes = [C.c_void_p, C.c_int32, C.POINTER(C.c_size_t)]
    lib.qkv_project_workspace.restype = C.c_int32
    lib.wave_attn_chain.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(KvCache),
                                    C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p,
                                    C.c_float, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.wave_attn_chain.restype = C.c_int32
    lib.qkv_project.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(KvCache), C.c_void_p, C.c_int32,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.qkv_project.restype = C.c_int32
    lib.chain_store.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.chain_store.restype = C.c_int32
    lib.wave_last_error.argtypes = []
    lib.wave_last_error.restype = C.c_char_p
    _lib = lib
    return lib


class WaveError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def check(code: int) -> None:
    if code != WAVE_OK:
        raise WaveError(code, load().wave_last_error().decode())
