"""Pins for the oracle's sparse MQA-mode MLA ("详解DSA" Eq.(2); the mask-based
MLA forward of the same page; MQA mode as on the charlestar and luowle pages).

P1: the gather formulation equals the page's dense mask formulation
(``-inf`` everywhere except the selected columns, fp32-or-better softmax).
P2: with k >= pos+1 nothing is dropped, so DSA equals dense causal attention.
P5: closed forms (position 0, k = 1, identical values, convexity) and the
log-sum-exp against scipy.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import dsa_forward, sparse_mla, query_positions
from synth import standard_workload, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_case.json")


def test_hand_case_attention():
    g = json.load(open(GOLDEN))
    q = np.array(g["q_mla"], np.float32)
    kv = np.array(g["kv"], np.float32)
    idx = np.array(g["top2"])
    out, lse = sparse_mla(q, "f32", kv, "f32", idx, g["seq_lens"], g["q_len"],
                          math.log(3.0), dv=g["dv"])
    assert np.allclose(out, np.array(g["out_top2"], float), rtol=1e-14, atol=1e-13)
    assert np.allclose(np.exp(lse), np.array(g["lse_top2_exp"], float), rtol=1e-14)


def _dense_masked(q, kv, allowed, sm, dv):
    """The page's mask formulation: scores over every cache row, -inf where
    not allowed, softmax over the row, times V."""
    z = sm * (q.astype(np.float64) @ kv.astype(np.float64).T)      # [H, S]
    z = np.where(allowed[None, :], z, -np.inf)
    p = softmax(z, axis=1)
    return p @ kv[:, :dv].astype(np.float64), logsumexp(z, axis=1)


def test_gather_equals_dense_mask_formulation():
    rng = np.random.default_rng(12)
    B, q_len, S, H, D, dv, k = 2, 3, 40, 4, 24, 16, 9
    seq_lens = [40, 25]
    q = rng.standard_normal((B * q_len, H, D)).astype(np.float32)
    kv = rng.standard_normal((B, S, D)).astype(np.float32)
    _, pos = query_positions(seq_lens, q_len)
    idx = np.full((B * q_len, k), -1)
    for t in range(B * q_len):
        m = min(k, pos[t] + 1) - (t % 2)          # some rows not full
        idx[t, :m] = rng.choice(pos[t] + 1, m, replace=False)
        rng.shuffle(idx[t])                        # -1 anywhere, any order
    out, lse = sparse_mla(q, "f32", kv, "f32", idx, seq_lens, q_len, 0.3, dv=dv)
    for t in range(B * q_len):
        allowed = np.zeros(S, bool)
        allowed[idx[t][idx[t] >= 0]] = True
        o, l = _dense_masked(q[t], kv[t // q_len], allowed, 0.3, dv)
        assert np.allclose(out[t], o, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[t], l, rtol=1e-12)


def test_dsa_equals_dense_causal_when_nothing_is_dropped():
    """Rows with pos+1 <= k keep every valid key: DSA == dense causal MLA."""
    w = make_workload("small", 1, 48, 48, 48, 64, 4, fp8=False, seed=5)
    qi, ww, (ki, ks), qm, kv = w.qi(), w.w(), w.ki_all(), w.qm(), w.kv_all()
    idx, tau, out, lse, _ = dsa_forward(qi, "f32", ww, "f32", ki, "f32", qm, "f32",
                                        kv, "f32", w.seq_lens, w.q_len, w.topk, 0.25)
    for t in range(48):
        assert tau[t] == -np.inf and [int(i) for i in idx[t] if i >= 0] == list(range(t + 1))
        allowed = np.arange(48) <= t
        o, l = _dense_masked(qm[t], kv[0], allowed, 0.25, 512)
        assert np.allclose(out[t], o, rtol=1e-12, atol=1e-12)


def test_tiny_config_first_rows_are_dense():
    """The tiny 512-token configuration: rows t < 64 keep everything (k = 64)."""
    w = standard_workload("tiny512")
    rows = np.array([0, 1, 31, 63, 64, 300])
    qi, ww, (ki, ks), qm, kv = w.qi(), w.w(), w.ki_all(), w.qm(), w.kv_all()
    idx, tau, out, lse, _ = dsa_forward(qi, "f32", ww, "f32", ki, "f32", qm, "f32", kv,
                                        "f32", w.seq_lens, w.q_len, w.topk, w.sm_scale,
                                        rows=rows)
    for r, t in enumerate(rows[:4]):
        o, _ = _dense_masked(qm[t], kv[0], np.arange(512) <= t, w.sm_scale, 512)
        assert np.allclose(out[r], o, rtol=1e-12, atol=1e-12)
    assert np.all(idx[4:] >= 0) and tau[4] > -np.inf


def test_closed_forms():
    rng = np.random.default_rng(13)
    S, H, D, dv = 10, 3, 12, 8
    kv = rng.standard_normal((1, S, D)).astype(np.float32)
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    # position 0 sees only entry 0: out = V[0] exactly
    idx = np.full((S, 4), -1)
    idx[0, 2] = 0
    out, lse = sparse_mla(q, "f32", kv, "f32", idx, [S], S, 1.0, dv=dv)
    assert np.array_equal(out[0], np.broadcast_to(kv[0, 0, :dv].astype(np.float64), (H, dv)))
    assert np.allclose(lse[0], (q[0].astype(np.float64) @ kv[0, 0].astype(np.float64)))
    # a single selected entry gives its value row exactly
    idx1 = np.full((S, 1), -1)
    idx1[:, 0] = [min(t, 3) for t in range(S)]
    out1, _ = sparse_mla(q, "f32", kv, "f32", idx1, [S], S, 1.0, dv=dv)
    for t in range(S):
        assert np.array_equal(out1[t], np.broadcast_to(kv[0, min(t, 3), :dv].astype(np.float64), (H, dv)))
    # identical value rows: output equals that row whatever the weights
    kv2 = kv.copy()
    kv2[0, :, :dv] = kv2[0, 5, :dv]
    idx2 = np.array([[s for s in range(t + 1)] + [-1] * (S - t - 1) for t in range(S)])
    out2, _ = sparse_mla(q, "f32", kv2, "f32", idx2, [S], S, 0.7, dv=dv)
    assert np.allclose(out2, kv2[0, 5, :dv].astype(np.float64), rtol=1e-13, atol=1e-13)
    # convexity: each output coordinate within [min, max] of the selected values
    out3, _ = sparse_mla(q, "f32", kv, "f32", idx2, [S], S, 0.7, dv=dv)
    for t in range(S):
        v = kv[0, :t + 1, :dv].astype(np.float64)
        assert np.all(out3[t] >= v.min(axis=0) - 1e-12) and np.all(out3[t] <= v.max(axis=0) + 1e-12)


def test_empty_selection_and_bad_indices():
    q = np.ones((2, 1, 4), np.float32)
    kv = np.ones((1, 2, 4), np.float32)
    out, lse = sparse_mla(q, "f32", kv, "f32", np.array([[-1, -1], [0, 1]]), [2], 2, 1.0, dv=2)
    assert np.array_equal(out[0], np.zeros((1, 2))) and lse[0, 0] == -np.inf
    with pytest.raises(ValueError):
        sparse_mla(q, "f32", kv, "f32", np.array([[1, -1], [0, 1]]), [2], 2, 1.0, dv=2)
    with pytest.raises(ValueError):
        sparse_mla(q, "f32", kv, "f32", np.array([[0, -1], [1, 1]]), [2], 2, 1.0, dv=2)


def test_order_of_indices_does_not_matter():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 2, 8)).astype(np.float32)
    kv = rng.standard_normal((1, 30, 8)).astype(np.float32)
    sel = rng.choice(30, 12, replace=False)
    a, la = sparse_mla(q, "f32", kv, "f32", sel[None], [30], 1, 0.5, dv=4)
    b, lb = sparse_mla(q, "f32", kv, "f32", np.sort(sel)[None], [30], 1, 0.5, dv=4)
    assert np.allclose(a, b, rtol=1e-14) and np.allclose(la, lb, rtol=1e-14)
