"""Pins of the toy denoiser chain oracle (``oracle.chain``), CPU only.

* The projection against a brute-force triple loop with an explicit RMS.
* Its invariance to the input scale (a dropped normalisation fails it).
* The whole chain in a closed form: with W_q = 0 every score is 0, so each
  query row of a node is the plain mean of the V rows of its context, and with
  W_v = I those V rows are bf16(a / rms(a)) of the writer's own input.  The
  expected outputs are built by direct accumulation over the slots the
  progressive policy (design-space paper, Table 1: phi(j, r) = max(j - r, 0))
  selects, written out here independently of ``oracle.plan``.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import chain as oc
from oracle import plan as op
from oracle.attention import round_to_bf16


def bf16(x):
    return round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def test_project_matches_brute_force():
    rng = np.random.default_rng(5)
    heads, hd = 2, 3
    D = heads * hd
    a = bf16(rng.standard_normal((4, D)))
    w = bf16(rng.standard_normal((3 * D, D)) / math.sqrt(D))
    q, k, v = oc.project(a, w, heads, hd)
    got = np.concatenate([q.reshape(4, D), k.reshape(4, D), v.reshape(4, D)], axis=1)
    for t in range(4):
        ss = 0.0
        for c in range(D):
            ss += a[t, c] * a[t, c]
        r = math.sqrt(ss / D + 1e-6)
        for o in range(3 * D):
            acc = 0.0
            for c in range(D):
                acc += a[t, c] * w[o, c]
            assert got[t, o] == bf16(acc / r)


def test_project_is_scale_invariant():
    rng = np.random.default_rng(6)
    a = bf16(rng.standard_normal((16, 8)))
    w = bf16(rng.standard_normal((24, 8)) / math.sqrt(8))
    base = oc.project(a, w, 2, 4)
    for s in (0.25, 2.0, 64.0):
        got = oc.project(bf16(a * s), w, 2, 4)
        for x, y in zip(base, got):
            np.testing.assert_allclose(x, y, rtol=2.0 ** -7, atol=0)


def _closed_form_chain(B, K, L, layers, D, noise):
    """Uniform-attention chain, serial order U(i,K..1) then R(i): expected results."""
    v_slot = {}  # (layer, chunk, level) -> V rows [L, D]
    results = {}
    for i in range(B):
        a = noise(i)
        for lv in list(range(K, 0, -1)) + [0]:
            for layer in range(layers):
                rms = np.sqrt(np.mean(a * a, axis=1) + 1e-6)
                v_slot[(layer, i, lv)] = bf16(a / rms[:, None])
                ctx = [(i - r, max(lv - r, 0)) for r in range(i, 0, -1)] + [(i, lv)]
                rows = np.concatenate([v_slot[(layer, c, l)] for (c, l) in ctx], axis=0)
                mean = rows.sum(axis=0) / rows.shape[0]
                a = bf16(np.repeat(mean[None, :], L, axis=0))
            results[(i, lv)] = a
    return results


@pytest.mark.parametrize("sched", [op.SERIAL, op.WAVE])
def test_chain_uniform_attention_closed_form(sched):
    B, K, L, heads, hd, layers = 3, 2, 5, 2, 2, 2
    D = heads * hd
    rng = np.random.default_rng(7)
    noise_tab = {i: bf16(rng.standard_normal((L, D))) for i in range(B)}
    weights = []
    for _ in range(layers):
        w = np.zeros((3 * D, D))
        w[D:2 * D] = bf16(rng.standard_normal((D, D)))  # K: irrelevant when Q = 0
        w[2 * D:] = np.eye(D)                           # V = bf16(a / rms(a))
        weights.append(w)
    p = op.Params(B, K, op.PROGRESSIVE, sched, -1, L, 0, 0)
    plan = op.oracle_plan(p)
    got = oc.chain_rollout(p, plan, layers, heads, hd, lambda c: noise_tab[c], lambda l: weights[l],
                           1.0 / math.sqrt(hd))
    want = _closed_form_chain(B, K, L, layers, D, lambda c: noise_tab[c])
    # the plan refreshes a chunk only when a later node reads its clean slot
    assert set(got) <= set(want) and {(i, lv) for i in range(B) for lv in range(1, K + 1)} <= set(got)
    for key, (res, per_layer) in got.items():
        assert len(per_layer) == layers
        np.testing.assert_allclose(res, want[key], rtol=2.0 ** -7, atol=1e-12, err_msg=str(key))


def test_chain_rejects_conditioning_and_short_queries():
    p = op.Params(2, 1, op.PROGRESSIVE, op.SERIAL, -1, 4, 3, 0)
    with pytest.raises(ValueError):
        oc.chain_rollout(p, op.oracle_plan(p), 1, 1, 2, None, None, 1.0)
    p = op.Params(2, 1, op.PROGRESSIVE, op.SERIAL, -1, 4, 0, 2)
    with pytest.raises(ValueError):
        oc.chain_rollout(p, op.oracle_plan(p), 1, 1, 2, None, None, 1.0)
