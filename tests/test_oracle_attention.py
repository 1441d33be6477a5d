"""Pins of the oracle's attention and rollout.

* bfloat16 rounding against torch's own float32 -> bfloat16 conversion.
* No mask: torch's scaled_dot_product_attention in fp64 (a library routine).
* Closed forms: zero keys give LSE = log(n) and O = mean(V); constant V gives
  O = V; a single key gives O = v and LSE = its score.
* Softmax rows sum to 1; key permutation invariance.
* Block causality (Wan-Streamer v0.2, Figure 1; Wave Forcing summary,
  mechanism paragraph): a progressive steady round equals one SDPA call over
  the concatenated slots with a lower block-triangular mask; a clean node
  equals SDPA over [(0,0) .. (i-1,0), (i,j)]; a single chunk is plain
  bidirectional attention.
* Causality invariance and sensitivity of the serial rollout.
"""
import numpy as np
import pytest
import torch

from oracle import plan as op
from oracle.attention import masked_attention, round_to_bf16, slot_mask, softmax_rows
from oracle.rollout import rollout


def rng(seed):
    return np.random.default_rng(seed)


def test_round_to_bf16_matches_torch():
    r = rng(0)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32) * 3,
        r.standard_normal(1000).astype(np.float32) * 1e-39,  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.3895314e38, -3.3895314e38,
                  3.4028235e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], np.float32),
    ])
    # exact ties in both parities
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_unmasked_matches_sdpa_fp64():
    r = rng(1)
    q = r.standard_normal((37, 24))
    k = r.standard_normal((53, 24))
    v = r.standard_normal((53, 16))
    scale = 1 / np.sqrt(24)
    o, lse = masked_attention(q, k, v, np.zeros((37, 53)), scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale)[0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    ref_lse = torch.logsumexp(torch.from_numpy(q @ k.T * scale), dim=1).numpy()
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def test_closed_forms():
    r = rng(2)
    v = r.standard_normal((40, 8))
    q = r.standard_normal((5, 8))
    o, lse = masked_attention(q, np.zeros((40, 8)), v, np.zeros((5, 40)), 0.3)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14)
    assert np.allclose(lse, np.log(40.0), atol=1e-14)
    c = r.standard_normal(8)
    o, _ = masked_attention(q, r.standard_normal((40, 8)), np.tile(c, (40, 1)), np.zeros((5, 40)), 0.3)
    assert np.allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)
    k1 = r.standard_normal((1, 8))
    o, lse = masked_attention(q, k1, v[:1], np.zeros((5, 1)), 0.7)
    assert np.allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-15)
    assert np.allclose(lse, 0.7 * (q @ k1.T)[:, 0], atol=1e-14)
    # a masked key contributes nothing
    m = np.zeros((5, 40))
    m[:, 10:] = -np.inf
    kk = r.standard_normal((40, 8))
    o_m, lse_m = masked_attention(q, kk, v, m, 0.5)
    o_c, lse_c = masked_attention(q, kk[:10], v[:10], np.zeros((5, 10)), 0.5)
    assert np.allclose(o_m, o_c, atol=1e-14) and np.allclose(lse_m, lse_c, atol=1e-14)


def test_rows_sum_to_one_and_permutation_invariance():
    r = rng(3)
    q = r.standard_normal((20, 16)) * 2
    k = r.standard_normal((70, 16)) * 2
    v = r.standard_normal((70, 16))
    m = np.zeros((20, 70))
    m[:, 50:] = -np.inf
    p = softmax_rows(q, k, m, 0.25)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    o, lse = masked_attention(q, k, v, m, 0.25)
    perm = r.permutation(70)
    o2, lse2 = masked_attention(q, k[perm], v[perm], m[:, perm], 0.25)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


def _inputs(B, K, L, h, d, seed, cond=0):
    r = rng(seed)
    store = {}

    def get_kv(c, lv):
        key = ("kv", c, lv)
        if key not in store:
            n = cond if lv == op.COND else L
            store[key] = (r.standard_normal((n, h, d)), r.standard_normal((n, h, d)))
        return store[key]

    def get_q(c, lv):
        key = ("q", c, lv)
        if key not in store:
            store[key] = r.standard_normal((L, h, d))
        return store[key]

    return get_q, get_kv, store


def _sdpa_blockmask(q, ks, vs, allowed, scale):
    """One fp64 SDPA call over concatenated key blocks with a boolean block mask."""
    kcat = np.concatenate(ks, axis=0)
    vcat = np.concatenate(vs, axis=0)
    cols = np.concatenate([np.full(k.shape[0], a) for k, a in zip(ks, allowed)])
    mask = torch.from_numpy(np.broadcast_to(cols, (q.shape[0], kcat.shape[0])).copy())
    out = []
    for h in range(q.shape[1]):
        out.append(torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None], torch.from_numpy(kcat[:, h])[None],
            torch.from_numpy(vcat[:, h])[None], attn_mask=mask[None], scale=scale)[0].numpy())
    return np.stack(out, axis=1)


def test_progressive_steady_round_is_block_causal_sdpa():
    B, K, L, h, d = 6, 3, 8, 2, 8
    p = op.Params(B, K, op.PROGRESSIVE, op.WAVE, -1, L, 0)
    pl = op.oracle_plan(p)
    get_q, get_kv, _ = _inputs(B, K, L, h, d, 4)
    scale = 1 / np.sqrt(d)
    out = rollout(p, pl, get_q, get_kv, scale)
    t = 4  # steady round: chunks t-K .. t in flight
    # Key sequence: (0,0)..(t-K,0), then (t-K+1,1) .. (t,K); query blocks are
    # the last K+1 chunks, query chunk c sees key blocks 0..c.
    seq = [(c, 0) for c in range(0, t - K + 1)] + [(t - K + m, m) for m in range(1, K + 1)]
    ks = [get_kv(*s)[0] for s in seq]
    vs = [get_kv(*s)[1] for s in seq]
    for c in range(t - K, t + 1):
        lv = 0 if c == t - K else c - (t - K)
        allowed = [i <= c for i in range(len(seq))]
        ref = _sdpa_blockmask(get_q(c, lv), ks, vs, allowed, scale)
        assert np.max(np.abs(out[(c, lv)][0] - ref)) < 1e-12


def test_clean_node_is_block_causal_sdpa():
    B, K, L, h, d = 4, 2, 8, 2, 8
    p = op.Params(B, K, op.CLEAN, op.WAVE, -1, L, 0)
    pl = op.oracle_plan(p)
    get_q, get_kv, _ = _inputs(B, K, L, h, d, 5)
    scale = 1 / np.sqrt(d)
    out = rollout(p, pl, get_q, get_kv, scale)
    for i in range(B):
        for j in range(1, K + 1):
            seq = [(c, 0) for c in range(i)] + [(i, j)]
            ref = _sdpa_blockmask(get_q(i, j), [get_kv(*s)[0] for s in seq],
                                  [get_kv(*s)[1] for s in seq], [True] * len(seq), scale)
            assert np.max(np.abs(out[(i, j)][0] - ref)) < 1e-12


@pytest.mark.parametrize("policy", [op.CLEAN, op.SAME_LEVEL, op.PROGRESSIVE])
def test_single_chunk_is_full_attention(policy):
    for B, H in ((1, -1), (4, 0)):
        p = op.Params(B, 2, policy, op.WAVE, H, 12, 0)
        pl = op.oracle_plan(p)
        get_q, get_kv, _ = _inputs(B, 2, 12, 2, 8, 6)
        out = rollout(p, pl, get_q, get_kv, 0.35)
        for (c, lv), (o, lse) in out.items():
            k, v = get_kv(c, lv)
            ref = _sdpa_blockmask(get_q(c, lv), [k], [v], [True], 0.35)
            assert np.max(np.abs(o - ref)) < 1e-12


def test_rollout_causality_invariance_and_sensitivity():
    B, K, L, h, d = 5, 3, 8, 2, 8
    p = op.Params(B, K, op.PROGRESSIVE, op.WAVE, -1, L, 4)
    pl = op.oracle_plan(p)
    get_q, get_kv, store = _inputs(B, K, L, h, d, 7, cond=4)
    base = rollout(p, pl, get_q, get_kv, 0.3)
    # Perturb every slot of chunks > 2: outputs of chunks <= 2 are unchanged.
    for key in list(store):
        if key[0] == "kv" and key[1] > 2:
            k, v = store[key]
            store[key] = (k + 5.0, v - 3.0)
    pert = rollout(p, pl, get_q, get_kv, 0.3)
    for (c, lv), (o, lse) in base.items():
        same = np.array_equal(o, pert[(c, lv)][0]) and np.array_equal(lse, pert[(c, lv)][1])
        if c <= 2:
            assert same
        else:
            assert not same
    # Sensitivity: perturbing one in-context slot changes the reader.
    k, v = store[("kv", 0, op.COND)]
    store[("kv", 0, op.COND)] = (k, v + 1.0)
    pert2 = rollout(p, pl, get_q, get_kv, 0.3)
    assert np.max(np.abs(pert2[(1, 3)][0] - pert[(1, 3)][0])) > 1e-3
    # Chunk 0 reads its own conditioning slot, so it moves too.
    assert np.max(np.abs(pert2[(0, 3)][0] - pert[(0, 3)][0])) > 1e-3


def test_rollout_rejects_unwritten_read():
    p = op.Params(3, 2, op.PROGRESSIVE, op.WAVE, -1, 4, 0)
    pl = op.oracle_plan(p)
    # Drop the refresh of chunk 0 from the plan: the round that needs (0,0) fails.
    bad = dict(pl)
    get_q, get_kv, _ = _inputs(3, 2, 4, 1, 4, 8)
    nodes = list(pl["nodes"])
    for idx, n in enumerate(nodes):
        if n[2] == op.REFRESH and n[0] == 0:
            nodes[idx] = n[:8] + (n[8], 0)  # no writes
    bad["nodes"] = nodes
    with pytest.raises(RuntimeError):
        rollout(p, bad, get_q, get_kv, 0.5)
