"""Pins of the indexer KL objective oracle (``oracle.indexer_kl``):

* scipy's ``entropy(p, q)`` (relative entropy) on the distributions built
  step by step from Eq.(3) and Eq.(4);
* KL = 0 when the indexer reproduces the teacher (I = log v + const);
* Gibbs' inequality (KL >= 0) and the two-position closed form with one head;
* the sparse objective on a set that keeps every position equals the dense
  one; with exact normalisers every head's weights sum to one (v sums to H).
"""

import numpy as np
from scipy.stats import entropy

from oracle import attention_lse, indexer_kl, query_positions


def _inputs(rng, B, q_len, S, H):
    q = rng.standard_normal((B * q_len, H, 576)).astype(np.float32)
    kv = rng.standard_normal((B, S, 576)).astype(np.float32)
    scores = (rng.standard_normal((B * q_len, S)) * 2).astype(np.float32)
    return q, kv, scores


def test_matches_scipy_relative_entropy():
    rng = np.random.default_rng(1)
    B, q_len, S, H = 2, 3, 50, 4
    seq = np.array([50, 21])
    q, kv, scores = _inputs(rng, B, q_len, S, H)
    sm = 0.05
    lse = attention_lse(q, "f32", kv, "f32", None, seq, q_len, sm) + rng.standard_normal((B * q_len, H)) * 0.1
    kl, total = indexer_kl(q, "f32", kv, "f32", lse, scores, None, seq, q_len, sm)
    b, pos = query_positions(seq, q_len)
    for t in range(B * q_len):
        n = pos[t] + 1
        z = sm * q[t].astype(np.float64) @ kv[b[t], :n].astype(np.float64).T
        v = np.exp(z - lse[t][:, None]).sum(axis=0)
        ph = np.exp(scores[t, :n].astype(np.float64))
        assert abs(kl[t] - entropy(v, ph)) < 1e-10       # entropy normalises both arguments
    assert abs(total - kl.sum()) < 1e-12


def test_zero_when_indexer_matches_teacher_and_gibbs():
    rng = np.random.default_rng(2)
    B, q_len, S, H = 1, 4, 30, 3
    seq = np.array([30])
    q, kv, scores = _inputs(rng, B, q_len, S, H)
    sm = 0.04
    lse = attention_lse(q, "f32", kv, "f32", None, seq, q_len, sm)
    b, pos = query_positions(seq, q_len)
    teacher = np.full_like(scores, -50.0, dtype=np.float64)
    for t in range(q_len):
        n = pos[t] + 1
        z = sm * q[t].astype(np.float64) @ kv[0, :n].astype(np.float64).T
        v = np.exp(z - lse[t][:, None]).sum(axis=0)
        assert abs(v.sum() - H) < 1e-9                    # exact normalisers: each head sums to one
        teacher[t, :n] = np.log(v) + 3.7                  # any constant shift
    kl, _ = indexer_kl(q, "f32", kv, "f32", lse, teacher, None, seq, q_len, sm)
    assert np.all(np.abs(kl) < 1e-12)
    kl_rand, _ = indexer_kl(q, "f32", kv, "f32", lse, scores, None, seq, q_len, sm)
    assert np.all(kl_rand > 0)


def test_two_positions_one_head_closed_form():
    # p = (sigma(d), 1 - sigma(d)) with d = z0 - z1; p_hat likewise with e = I0 - I1
    rng = np.random.default_rng(3)
    q, kv, scores = _inputs(rng, 1, 1, 2, 1)
    sm = 0.03
    seq = np.array([2])
    lse = np.array([[0.7]])                               # any normaliser: Eq.(3) renormalises
    kl, _ = indexer_kl(q, "f32", kv, "f32", lse, scores, None, seq, 1, sm)
    z = sm * kv[0].astype(np.float64) @ q[0, 0].astype(np.float64)
    p0 = 1 / (1 + np.exp(z[1] - z[0]))
    h0 = 1 / (1 + np.exp(float(scores[0, 1]) - float(scores[0, 0])))
    want = p0 * np.log(p0 / h0) + (1 - p0) * np.log((1 - p0) / (1 - h0))
    assert abs(kl[0] - want) < 1e-12


def test_sparse_on_full_set_equals_dense_and_set_handling():
    rng = np.random.default_rng(4)
    B, q_len, S, H = 2, 2, 40, 2
    seq = np.array([40, 9])
    q, kv, scores = _inputs(rng, B, q_len, S, H)
    sm = 0.05
    lse = attention_lse(q, "f32", kv, "f32", None, seq, q_len, sm)
    dense, _ = indexer_kl(q, "f32", kv, "f32", lse, scores, None, seq, q_len, sm)
    _, pos = query_positions(seq, q_len)
    idx = np.full((B * q_len, 64), -1, np.int32)
    for t in range(B * q_len):
        perm = rng.permutation(pos[t] + 1)               # order does not matter; -1 and > pos are skipped
        idx[t, :len(perm)] = perm
        idx[t, len(perm):len(perm) + 2] = [pos[t] + 1, S + 3]
    sparse, _ = indexer_kl(q, "f32", kv, "f32", lse, scores, idx, seq, q_len, sm)
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-12)
    # a strict subset gives the KL of the renormalised restrictions
    sub = np.full_like(idx, -1)
    sub[:, :5] = np.arange(5)
    kl_sub, _ = indexer_kl(q, "f32", kv, "f32", lse, scores, sub, seq, q_len, sm)
    b, _ = query_positions(seq, q_len)
    for t in range(B * q_len):
        z = sm * q[t].astype(np.float64) @ kv[b[t], :5].astype(np.float64).T
        v = np.exp(z - lse[t][:, None]).sum(axis=0)
        assert abs(kl_sub[t] - entropy(v, np.exp(scores[t, :5].astype(np.float64)))) < 1e-10
