"""Native planner (libwave.so, through the C ABI) against the brute-force oracle.

Plans, gather lists, write lists and physical slots must match bit-exactly;
the work list and the descriptor are checked for their own invariants.
Runs on the CPU: wave_plan is host code.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from block_causal_attention_wave_amd import _lib
import block_causal_attention_wave_amd as wv
from oracle import plan as op
from wave_inputs import WORKLOADS

import test_oracle_plan as worked  # hand-worked plan fixtures and their checker

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def native(B, K, policy, sched, H=-1, L=16, cond=0, q_tile=0, query_len=0):
    return wv.wave_plan(B=B, K=K, policy=policy, sched=sched, history_cap=H, chunk_len=L,
                        cond_len=cond, q_tile=q_tile, query_len=query_len)


def assert_same(pn, po):
    assert pn.num_rounds == po["num_rounds"]
    assert pn.num_phys_slots == po["num_phys_slots"]
    assert pn.round_node_begin.tolist() == po["round_node_begin"]
    assert [tuple(x) for x in pn.nodes.tolist()] == [tuple(x) for x in po["nodes"]]
    assert [tuple(x) for x in pn.ctx.tolist()] == [tuple(x) for x in po["ctx"]]
    assert [tuple(x) for x in pn.writes.tolist()] == [tuple(x) for x in po["writes"]]


GRID = [(B, K, pol, sch, H, cond)
        for B in (1, 2, 3, 5, 7, 12)
        for K in (1, 2, 3, 4, 6)
        for pol in (op.CLEAN, op.SAME_LEVEL, op.PROGRESSIVE)
        for sch in (op.SERIAL, op.WAVE)
        for H in (-1, 0, 1, 2, 6)
        for cond in (0, 1)]


@pytest.mark.parametrize("B,K,pol,sch,H,cond", GRID)
def test_planner_matches_oracle_grid(B, K, pol, sch, H, cond):
    L, C_ = 48, (17 if cond else 0)
    pn = native(B, K, pol, sch, H, L, C_)
    po = op.oracle_plan(op.Params(B, K, pol, sch, H, L, C_))
    assert_same(pn, po)


@pytest.mark.parametrize("key", sorted(WORKLOADS))
def test_planner_matches_oracle_workloads(key):
    w = WORKLOADS[key]
    for pol in w.policies:
        for sch in (op.SERIAL, op.WAVE):
            pn = native(w.B, w.K, pol, sch, w.history_cap, w.chunk_len, w.cond_len)
            po = op.oracle_plan(op.Params(w.B, w.K, pol, sch, w.history_cap, w.chunk_len, w.cond_len))
            assert_same(pn, po)


@pytest.mark.parametrize("query_len", [1, 64, 100, 300])
@pytest.mark.parametrize("pol", [op.CLEAN, op.SAME_LEVEL, op.PROGRESSIVE])
def test_planner_query_len_matches_oracle(query_len, pol):
    """Short query chunks (the decode-shaped case) change only row offsets."""
    pn = native(6, 3, pol, op.WAVE, -1, 200, 33, query_len=query_len)
    po = op.oracle_plan(op.Params(6, 3, pol, op.WAVE, -1, 200, 33, query_len))
    assert_same(pn, po)
    assert (pn.nodes[:, 5] == query_len).all()
    for t in range(pn.num_rounds):
        nb, ne = pn.round_node_begin[t], pn.round_node_begin[t + 1]
        assert pn.round_q_rows[t] == query_len * (ne - nb)
        items = pn.work[pn.round_work_begin[t]:pn.round_work_begin[t + 1]]
        assert int(items[:, 2].sum()) == query_len * (ne - nb)


@pytest.mark.parametrize("name", sorted(worked.PLAN_FIXTURES))
def test_planner_matches_worked_plans(name):
    """The native planner reproduces every hand-worked plan fixture."""
    prm = worked.PLAN_FIXTURES[name][0]
    pn = native(prm.B, prm.K, prm.policy, prm.sched, prm.history_cap, prm.chunk_len, prm.cond_len)
    pl = {"num_rounds": pn.num_rounds, "num_phys_slots": pn.num_phys_slots,
          "nodes": [tuple(x) for x in pn.nodes.tolist()], "ctx": [tuple(x) for x in pn.ctx.tolist()],
          "writes": [tuple(x) for x in pn.writes.tolist()]}
    worked.check_plan_fixture(name, pl)


def test_workload_capacities_and_rounds():
    """Round counts and slot capacities of the named workloads."""
    cases = {
        (7, 4, op.PROGRESSIVE, -1): (10, 7),
        (7, 5, op.PROGRESSIVE, -1): (11, 7),
        (7, 5, op.SAME_LEVEL, -1): (11, 25),
        (7, 5, op.CLEAN, -1): (35, 7),
        (28, 4, op.PROGRESSIVE, 6): (31, 11),
        (4, 2, op.PROGRESSIVE, -1): (5, 4),
    }
    for (B, K, pol, H), (R, cap) in cases.items():
        pn = native(B, K, pol, op.WAVE, H, 4680)
        assert (pn.num_rounds, pn.num_phys_slots) == (R, cap)
    pn = native(8, 2, op.SAME_LEVEL, op.WAVE, -1, 2824, 512)
    assert (pn.num_rounds, pn.num_phys_slots) == (9, 23)


def test_work_list_covers_nodes_and_is_sorted():
    pn = native(7, 4, op.PROGRESSIVE, op.WAVE, -1, 4680, 0)
    assert pn.q_tile == 256
    for t in range(pn.num_rounds):
        items = pn.work[pn.round_work_begin[t]:pn.round_work_begin[t + 1]]
        nb, ne = pn.round_node_begin[t], pn.round_node_begin[t + 1]
        cover = {}
        for node, q0, qr, keys in items.tolist():
            assert nb <= node < ne
            n = pn.nodes[node]
            assert 0 < qr <= 256 and q0 % 256 == 0 and q0 + qr <= n[5]
            assert keys == int(pn.node_ctx(n)[:, 3].sum())
            cover.setdefault(node, []).append((q0, qr))
        for node in range(nb, ne):
            rows = sorted(cover[node])
            assert rows[0][0] == 0 and sum(r for _, r in rows) == pn.nodes[node][5]
        tiles = [int(np.ceil(pn.node_ctx(pn.nodes[it[0]])[:, 3] / 64).sum()) for it in items]
        assert tiles == sorted(tiles, reverse=True)


def test_descriptor_layout():
    pn = native(5, 3, op.PROGRESSIVE, op.WAVE, 2, 100, 7)
    d = pn.desc()
    assert d[0] == 0x57415645 and d[1] == 2
    nr, nn, nc, nw, nk = d[2:7]
    assert (nr, nn, nc, nw, nk) == (pn.num_rounds, len(pn.nodes), len(pn.ctx), len(pn.writes), len(pn.work))
    off_r, off_n, off_c, off_w, off_k = d[7:12]
    rt = d[off_r:off_r + 8 * nr].reshape(nr, 8)
    assert rt[:, 0].tolist() == pn.round_node_begin[:-1].tolist()
    assert rt[:, 6].tolist() == pn.round_q_rows.tolist()
    assert rt[:, 7].tolist() == pn.round_src_rows.tolist()
    nt = d[off_n:off_n + 6 * nn].reshape(nn, 6)
    assert (nt[:, 0] == pn.nodes[:, 4]).all() and (nt[:, 3] == pn.nodes[:, 7]).all()
    assert (nt[:, 4] == pn.nodes[:, 0]).all() and (nt[:, 5] == pn.nodes[:, 1]).all()
    ct = d[off_c:off_c + 2 * nc].reshape(nc, 2)
    assert (ct[:, 0] == pn.ctx[:, 2]).all() and (ct[:, 1] == pn.ctx[:, 3]).all()
    wt = d[off_w:off_w + 4 * nw].reshape(nw, 4)
    for t in range(nr):
        w0, w1 = pn.round_write_begin[t], pn.round_write_begin[t + 1]
        assert wt[w0:w1, 2].tolist() == np.concatenate([[0], np.cumsum(pn.writes[w0:w1, 3])[:-1]]).tolist()
    assert len(d) == off_k + 4 * nk
    # deterministic
    assert np.array_equal(d, native(5, 3, op.PROGRESSIVE, op.WAVE, 2, 100, 7).desc())


@pytest.mark.parametrize("bad", [
    dict(B=0), dict(K=0), dict(policy=3), dict(sched=2), dict(history_cap=-2),
    dict(chunk_len=0), dict(cond_len=-1), dict(q_tile=-1),
])
def test_invalid_params_rejected(bad):
    kw = dict(B=3, K=2, policy=0, sched=1, history_cap=-1, chunk_len=8, cond_len=0, q_tile=0)
    kw.update(bad)
    with pytest.raises(wv.WaveError) as e:
        wv.wave_plan(**kw)
    assert e.value.code == _lib.WAVE_ERR_INVALID_ARG
    assert "wave_plan" in str(e.value)


def test_abi_exports_every_header_symbol():
    with open(os.path.join(ROOT, "include", "wave.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"^\s*(?:int32_t|void|const char\*)\s+(\w+)\(", hdr, re.M))
    assert declared == set(_lib.EXPORTS)
    lib = C.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_device_calls_validate_before_launch():
    """Errors that must be caught on the host, before any launch (no GPU needed)."""
    lib = _lib.load()
    pn = native(4, 2, op.PROGRESSIVE, op.WAVE, -1, 128, 0)
    fake = C.c_void_p(0x10000)  # never dereferenced: validation fails first
    cache = _lib.KvCache(0x10000, 0x20000, 4, 2, 64, 128)
    stream = C.c_void_p(0)

    def attn(round_=0, cache_=cache, q=fake, qd=0, stride=128, scale=0.125, desc=fake):
        return lib.wave_attn(pn.handle, desc, round_, C.byref(cache_), q, qd, stride, fake, None,
                             scale, None, 0, stream)

    assert attn(round_=5) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(round_=-1) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(desc=None) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(q=None) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(qd=7) == _lib.WAVE_ERR_UNSUPPORTED
    assert attn(stride=64) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(scale=float("nan")) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(cache_=_lib.KvCache(0x10000, 0x20000, 3, 2, 64, 128)) == _lib.WAVE_ERR_CAPACITY
    assert attn(cache_=_lib.KvCache(0x10000, 0x20000, 4, 2, 64, 64)) == _lib.WAVE_ERR_CAPACITY
    assert attn(cache_=_lib.KvCache(0x10000, 0x20000, 4, 2, 96, 128)) == _lib.WAVE_ERR_UNSUPPORTED
    assert attn(cache_=_lib.KvCache(0x10000, 0x20000, 4, 2, 64, 100)) == _lib.WAVE_ERR_INVALID_ARG
    assert attn(cache_=_lib.KvCache(0, 0x20000, 4, 2, 64, 128)) == _lib.WAVE_ERR_INVALID_ARG
    # wave_attn_chain: wave_attn's checks, then a 4-byte aligned row_sq
    assert lib.wave_attn_chain(pn.handle, fake, 5, C.byref(cache), fake, 0, 128, fake, None, 0.125, fake, None, 0,
                               stream) == _lib.WAVE_ERR_INVALID_ARG
    assert lib.wave_attn_chain(pn.handle, fake, 0, C.byref(cache), fake, 0, 128, fake, None, 0.125,
                               C.c_void_p(0x10002), None, 0, stream) == _lib.WAVE_ERR_UNSUPPORTED
    # 32-bit per-lane V^T tile offsets: (head_dim-1)*lpad*2 + 128 must fit in int32
    lim128 = (2**31 - 1 - 128) // (127 * 2) // 64 * 64
    lim64 = (2**31 - 1 - 128) // (63 * 2) // 64 * 64
    for hd, lim in ((128, lim128), (64, lim64)):
        pbig = _lib.KvCache(0x10000, 0x20000, 4, 2, hd, lim + 64)
        assert lib.wave_attn(pn.handle, fake, 0, C.byref(pbig), fake, 0, 2 * hd, fake, None, 0.1, None, 0,
                             stream) == _lib.WAVE_ERR_UNSUPPORTED
        assert b"32-bit" in lib.wave_last_error()
        assert lib.kv_write(pn.handle, fake, 0, C.byref(pbig), fake, fake, 0, 2 * hd,
                            stream) == _lib.WAVE_ERR_UNSUPPORTED
        # the largest accepted lpad passes this check (and fails later, on the null q)
        ok = _lib.KvCache(0x10000, 0x20000, 4, 2, hd, lim)
        assert lib.wave_attn(pn.handle, fake, 0, C.byref(ok), None, 0, 2 * hd, fake, None, 0.1, None, 0,
                             stream) == _lib.WAVE_ERR_INVALID_ARG
        assert b"null q" in lib.wave_last_error()
    assert b"capacity" in lib.wave_last_error() or len(lib.wave_last_error()) > 0
    pn128 = native(4, 2, op.PROGRESSIVE, op.WAVE, -1, 128, 0, q_tile=128)
    assert lib.wave_attn(pn128.handle, fake, 0, C.byref(cache), fake, 0, 128, fake, None, 0.1,
                         None, 0, stream) == _lib.WAVE_ERR_UNSUPPORTED

    # split-KV: workspace checks
    def split(ws=fake, nbytes=1 << 30, splits=2):
        return lib.wave_attn_splitkv(pn.handle, fake, 0, C.byref(cache), fake, 0, 128, fake, None, 0.1,
                                     splits, ws, nbytes, stream)

    assert split(ws=None) == _lib.WAVE_ERR_INVALID_ARG
    assert split(ws=C.c_void_p(0x10010)) == _lib.WAVE_ERR_INVALID_ARG  # not 256-byte aligned
    assert split(nbytes=16) == _lib.WAVE_ERR_CAPACITY
    assert split(splits=-1) == _lib.WAVE_ERR_INVALID_ARG
    b, s = C.c_size_t(), C.c_int32()
    assert lib.wave_attn_splitkv_workspace(pn.handle, 0, 2, 64, 3, C.byref(b), C.byref(s)) == 0
    assert s.value == 3 and b.value >= 3 * 128 * 2 * 64 * 4 + 3 * 2 * 128 * 4
    assert lib.wave_attn_splitkv_workspace(pn.handle, 9, 2, 64, 3, C.byref(b), C.byref(s)) != 0

    # allocation-free split-KV: a split count whose partials exceed the
    # library's scratch is refused before any launch; so are bad arguments
    def noalloc(splits=2, q=fake):
        return lib.wave_attn_splitkv_noalloc(pn.handle, fake, 0, C.byref(cache), q, 0, 128, fake, None, 0.1,
                                             splits, stream)

    assert noalloc(q=None) == _lib.WAVE_ERR_INVALID_ARG
    assert noalloc(splits=-1) == _lib.WAVE_ERR_INVALID_ARG
    wide = native(3, 2, op.SAME_LEVEL, op.WAVE, -1, 4096, 0)
    wcache = _lib.KvCache(0x10000, 0x20000, wide.num_phys_slots, 40, 128, wide.lpad())
    b = C.c_size_t()
    assert lib.wave_attn_splitkv_workspace(wide.handle, 2, 40, 128, 4, C.byref(b), None) == 0
    assert b.value > _lib.WAVE_NOALLOC_SCRATCH_BYTES
    assert lib.wave_attn_splitkv_noalloc(wide.handle, fake, 2, C.byref(wcache), fake, 0, 40 * 128, fake, None,
                                         0.1, 4, stream) == _lib.WAVE_ERR_CAPACITY
    assert b"WAVE_NOALLOC_SCRATCH_BYTES" in lib.wave_last_error()

    def kvw(round_=0, src=fake, dt=0, stride=128):
        return lib.kv_write(pn.handle, fake, round_, C.byref(cache), src, src, dt, stride, stream)

    assert kvw(round_=9) == _lib.WAVE_ERR_INVALID_ARG
    assert kvw(src=None) == _lib.WAVE_ERR_INVALID_ARG
    assert kvw(dt=5) == _lib.WAVE_ERR_UNSUPPORTED
    assert kvw(stride=10) == _lib.WAVE_ERR_INVALID_ARG
    assert kvw(src=C.c_void_p(0x10008)) == _lib.WAVE_ERR_UNSUPPORTED


def test_wave_round_validates_every_layer_before_launch():
    """wave_round checks every layer's arguments on the host before it enqueues
    anything, and the error names the layer (no GPU needed: each call below
    has an invalid layer, so nothing is launched)."""
    lib = _lib.load()
    pn = native(4, 2, op.PROGRESSIVE, op.WAVE, -1, 128, 0)
    fake = 0x10000  # never dereferenced
    good = _lib.KvCache(0x10000, 0x20000, 4, 2, 64, 128)
    P = C.c_void_p * 2

    def rnd(n=2, caches=(good, good), k=(fake, fake), q=(fake, fake), o=(fake, fake), qd=0, round_=0,
            scale=0.125):
        arr = (_lib.KvCache * 2)(*caches)
        return lib.wave_round(pn.handle, C.c_void_p(fake), round_, n, arr, P(*k), P(fake, fake), 0, 128, P(*q), qd,
                              128, P(*o), None, scale, None, 0, C.c_void_p(0))

    assert rnd(n=0) == _lib.WAVE_ERR_INVALID_ARG
    assert lib.wave_round(pn.handle, C.c_void_p(fake), 0, 2, None, P(fake, fake), P(fake, fake), 0, 128,
                          P(fake, fake), 0, 128, P(fake, fake), None, 0.125, None, 0,
                          C.c_void_p(0)) == _lib.WAVE_ERR_INVALID_ARG
    assert rnd(q=(fake, 0)) == _lib.WAVE_ERR_INVALID_ARG and b"layer 1" in lib.wave_last_error()
    assert rnd(k=(fake, 0)) == _lib.WAVE_ERR_INVALID_ARG and b"layer 1" in lib.wave_last_error()
    assert rnd(o=(0, fake)) == _lib.WAVE_ERR_INVALID_ARG and b"layer 0" in lib.wave_last_error()
    short = _lib.KvCache(0x10000, 0x20000, 4, 2, 64, 64)
    assert rnd(caches=(good, short)) == _lib.WAVE_ERR_CAPACITY and b"layer 1" in lib.wave_last_error()
    assert rnd(round_=9) == _lib.WAVE_ERR_INVALID_ARG
    assert rnd(qd=7) == _lib.WAVE_ERR_UNSUPPORTED
    assert rnd(scale=float("inf")) == _lib.WAVE_ERR_INVALID_ARG


def test_tail_balancing_choice_and_workspace_checks():
    """wave_attn's tail balancing: the memoised choice for the Wan2.1-1.3B round-6
    shape (95 work items x 12 heads on 256 compute units) cuts some trailing
    items; a single compute unit never pays for a cut; the workspace size
    follows the documented layout; a misaligned or short workspace is rejected
    on the host before any launch."""
    lib = _lib.load()
    w = WORKLOADS[2]
    pn = native(w.B, w.K, op.PROGRESSIVE, op.WAVE, -1, w.chunk_len, 0)
    b, m, s = C.c_size_t(), C.c_int32(), C.c_int32()
    assert lib.wave_attn_workspace(pn.handle, w.round, w.heads, w.head_dim, 256, C.byref(b), C.byref(m),
                                   C.byref(s)) == 0
    items, splits = m.value, s.value
    assert 1 <= items <= 95 and 2 <= splits <= 4
    prows = items * 256
    o_bytes = (splits * prows * w.heads * w.head_dim * 4 + 255) // 256 * 256
    assert b.value == o_bytes + splits * w.heads * prows * 4
    again = C.c_size_t()
    assert lib.wave_attn_workspace(pn.handle, w.round, w.heads, w.head_dim, 256, C.byref(again), None,
                                   None) == 0
    assert again.value == b.value
    assert lib.wave_attn_workspace(pn.handle, w.round, w.heads, w.head_dim, 1, C.byref(again), C.byref(m),
                                   C.byref(s)) == 0
    assert again.value == 0 and m.value == 0
    for bad in ((w.round, 0, 128, 256), (w.round, 12, 96, 256), (w.round, 12, 128, -1), (99, 12, 128, 256)):
        assert lib.wave_attn_workspace(pn.handle, *bad, C.byref(again), None, None) == _lib.WAVE_ERR_INVALID_ARG

    # wave_attn itself (the device count falls back to 256 compute units without a GPU)
    cache = _lib.KvCache(0x10000, 0x20000, pn.num_phys_slots, w.heads, w.head_dim, pn.lpad())
    fake = C.c_void_p(0x10000)
    dev_cus = C.c_size_t()
    assert lib.wave_attn_workspace(pn.handle, w.round, w.heads, w.head_dim, 0, C.byref(dev_cus), None,
                                   None) == 0

    def attn(ws, nbytes):
        return lib.wave_attn(pn.handle, fake, w.round, C.byref(cache), fake, 0, w.heads * w.head_dim, fake,
                             None, 0.1, ws, nbytes, C.c_void_p(0))

    if dev_cus.value > 0:
        assert attn(C.c_void_p(0x10100), dev_cus.value - 1) == _lib.WAVE_ERR_CAPACITY
    assert attn(C.c_void_p(0x10010), 1 << 40) == _lib.WAVE_ERR_INVALID_ARG


def test_poisoned_slots_are_rewritten_before_any_later_read():
    """The GPU tests NaN-fill, after each round, the physical slots whose
    occupant no later round reads.  Over the capped-history long-video plan
    (B=28, K=4, H=6) such a slot is read again only after a rewrite, and the
    rolling cache does reuse slots."""
    from gpu_common import freed_after
    pn = native(28, 4, op.PROGRESSIVE, op.WAVE, 6, 16)
    freed = freed_after(pn)
    written = {t: {w[2] for w in pn.round_writes(t).tolist()} for t in range(pn.num_rounds)}
    reused = 0
    for t, slots in freed.items():
        for p in slots:
            for u in range(t + 1, pn.num_rounds):
                if p in written[u]:
                    reused += 1
                    break
                read = {e[2] for n in pn.round_nodes(u).tolist() for e in pn.node_ctx(n).tolist()}
                assert p not in read, (t, p, u)
    assert reused > 0 and pn.num_phys_slots < len(pn.writes)


@pytest.mark.parametrize("cond", [0, 512])
def test_capped_history_cache_does_not_grow_with_chunks(cond):
    """With a history cap the rolling cache's capacity is set by H and K, not by
    the video's length: B = 28 (the long-video workload) and B = 4000 need the
    same number of physical slots; the long plan keeps B+K-1 rounds and builds
    in well under the time of one round of attention."""
    import time
    short = native(28, 4, op.PROGRESSIVE, op.WAVE, 6, 4680, cond)
    t0 = time.perf_counter()
    long_ = native(4000, 4, op.PROGRESSIVE, op.WAVE, 6, 4680, cond)
    elapsed = time.perf_counter() - t0
    assert long_.num_rounds == 4000 + 4 - 1
    ref = op.oracle_plan(op.Params(28, 4, op.PROGRESSIVE, op.WAVE, 6, 4680, cond, 0))
    assert long_.num_phys_slots == short.num_phys_slots == ref["num_phys_slots"]
    if cond == 0:
        assert ref["num_phys_slots"] == 11  # the long-video workload's capacity per layer
    assert elapsed < 10.0


def test_splitkv_auto_split_count_fills_one_dispatch_wave():
    """num_splits = 0: the most splits whose workgroups (items x heads x splits)
    fit 256 compute units in one dispatch wave (the device count falls back to
    256 without a GPU), at most the longest item's key-tile count."""
    lib = _lib.load()
    w = WORKLOADS[6]
    pn = native(w.B, w.K, op.SAME_LEVEL, op.WAVE, w.history_cap, w.chunk_len, w.cond_len, query_len=w.query_len)
    items = int(pn.round_work_begin[w.round + 1] - pn.round_work_begin[w.round])
    b, s = C.c_size_t(), C.c_int32()
    assert lib.wave_attn_splitkv_workspace(pn.handle, w.round, w.heads, w.head_dim, 0, C.byref(b), C.byref(s)) == 0
    assert items == 2 and s.value == 256 // (items * w.heads) == 3
    # few key tiles: capped at the longest item's tile count
    small = native(2, 1, op.PROGRESSIVE, op.WAVE, -1, 100, 0, query_len=8)
    assert lib.wave_attn_splitkv_workspace(small.handle, 1, 1, 64, 0, C.byref(b), C.byref(s)) == 0
    assert s.value == 4  # round 1: R(0) and U(1,1); U(1,1) reads 2 slots of 2 key tiles
    # more workgroups than units: one split
    assert lib.wave_attn_splitkv_workspace(pn.handle, w.round, 200, w.head_dim, 0, C.byref(b), C.byref(s)) == 0
    assert s.value == 1


def test_chain_calls_validate_before_launch():
    """qkv_project / chain_store reject bad arguments on the host (no GPU needed)."""
    lib = _lib.load()
    pn = native(4, 2, op.PROGRESSIVE, op.WAVE, -1, 128, 0)
    fake = C.c_void_p(0x10000)
    ws = C.c_void_p(0x20000)
    cache = _lib.KvCache(0x10000, 0x20000, pn.num_phys_slots, 2, 64, pn.lpad())
    stream = C.c_void_p(0)
    b = C.c_size_t()
    assert lib.qkv_project_workspace(pn.handle, 1, C.byref(b)) == 0
    assert b.value == int(pn.round_q_rows[1]) * 4
    assert lib.qkv_project_workspace(pn.handle, 99, C.byref(b)) == _lib.WAVE_ERR_INVALID_ARG

    def proj(plan=pn, round_=1, cache_=cache, x=fake, layout=0, w=fake, q=fake, wsp=ws, nbytes=1 << 20, sq=None):
        return lib.qkv_project(plan.handle, fake, round_, C.byref(cache_), x, layout, sq, w, q, wsp, nbytes, stream)

    assert proj(round_=9) == _lib.WAVE_ERR_INVALID_ARG
    assert proj(x=None) == _lib.WAVE_ERR_INVALID_ARG
    assert proj(layout=2) == _lib.WAVE_ERR_INVALID_ARG
    assert proj(q=C.c_void_p(0x10008)) == _lib.WAVE_ERR_UNSUPPORTED
    assert proj(wsp=None) == _lib.WAVE_ERR_INVALID_ARG
    assert proj(nbytes=4) == _lib.WAVE_ERR_CAPACITY
    # per-head row statistics go with round-packed x only, and must be 4-byte aligned
    assert proj(layout=1, sq=C.c_void_p(0x30000)) == _lib.WAVE_ERR_INVALID_ARG
    assert proj(sq=C.c_void_p(0x30002)) == _lib.WAVE_ERR_UNSUPPORTED
    assert proj(cache_=_lib.KvCache(0x10000, 0x20000, pn.num_phys_slots, 1, 64, pn.lpad())) \
        == _lib.WAVE_ERR_UNSUPPORTED  # D = 64 is not a multiple of 128
    with_cond = native(4, 2, op.PROGRESSIVE, op.WAVE, -1, 128, 16)
    c2 = _lib.KvCache(0x10000, 0x20000, with_cond.num_phys_slots, 2, 64, with_cond.lpad())
    assert proj(plan=with_cond, cache_=c2) == _lib.WAVE_ERR_UNSUPPORTED
    short_q = native(4, 2, op.PROGRESSIVE, op.WAVE, -1, 128, 0, query_len=32)
    assert proj(plan=short_q) == _lib.WAVE_ERR_UNSUPPORTED

    def store(plan=pn, round_=1, dim=128, o=fake, st=fake):
        return lib.chain_store(plan.handle, fake, round_, dim, o, st, stream)

    assert store(round_=-1) == _lib.WAVE_ERR_INVALID_ARG
    assert store(dim=12) == _lib.WAVE_ERR_INVALID_ARG
    assert store(st=None) == _lib.WAVE_ERR_INVALID_ARG
    assert store(o=C.c_void_p(0x10004)) == _lib.WAVE_ERR_UNSUPPORTED
    assert store(plan=with_cond) == _lib.WAVE_ERR_UNSUPPORTED


def test_attention_rejects_gather_lists_past_512_slots():
    """The kernels stage a node's gather list in LDS, 512 slots at most: a plan
    whose longest list is 513 slots (513 chunks, clean history) is rejected on
    the host; 512 is accepted by the plan-level checks."""
    lib = _lib.load()
    fake = C.c_void_p(0x10000)
    for B, want in ((513, _lib.WAVE_ERR_UNSUPPORTED), (512, None)):
        pn = native(B, 1, op.CLEAN, op.WAVE, -1, 16, 0)
        assert int(pn.nodes[:, 7].max()) == B
        cache = _lib.KvCache(0x10000, 0x20000, pn.num_phys_slots, 1, 64, pn.lpad())
        misaligned_o = C.c_void_p(0x10008)  # fails a later host check, so nothing is launched
        rc = lib.wave_attn(pn.handle, fake, 0, C.byref(cache), fake, 0, 64, misaligned_o, None, 0.125,
                           None, 0, C.c_void_p(0))
        if want is not None:
            assert rc == want and b"512" in lib.wave_last_error()
        else:
            assert rc == _lib.WAVE_ERR_UNSUPPORTED and b"aligned" in lib.wave_last_error()
