"""Pins for the oracle's Lightning Indexer scores ("详解DSA" Eq.(1)).

Each test checks the oracle against something other than itself: a
hand-derived example, exact rational brute force, closed forms that reduce to
a plain matrix product, and invariants (positive homogeneity, masking,
isolation of sequences).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import indexer_scores, query_positions
from oracle.formats import decode_bf16, decode_e4m3fn
from synth.encode import encode_bf16_rne, encode_e4m3fn_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_case.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _num(x):
    return -np.inf if x == "-inf" else float(x)


def test_hand_case_scores():
    g = _golden()
    q = np.array(g["q_idx"], np.float32)
    w = np.array(g["w"], np.float32)
    k = np.array(g["k_idx"], np.float32)
    I = indexer_scores(q, "f32", w, "f32", k, "f32", g["seq_lens"], g["q_len"])
    exp = np.array([[_num(v) for v in row] for row in g["scores"]])
    assert np.array_equal(I, exp)


def test_query_positions_ragged():
    b, pos = query_positions([5, 3, 7], 2)
    assert b.tolist() == [0, 0, 1, 1, 2, 2]
    assert pos.tolist() == [3, 4, 1, 2, 5, 6]
    with pytest.raises(ValueError):
        query_positions([1], 2)


def _rand_fp8(rng, shape, spread=3.0):
    return encode_e4m3fn_rne(rng.standard_normal(shape) * spread)


def test_fp8_path_equals_exact_rational_brute_force():
    """Tiny fp8 case evaluated with Python Fractions, term by term."""
    rng = np.random.default_rng(3)
    HI, d, B, q_len, S = 3, 8, 2, 2, 5
    q = _rand_fp8(rng, (B * q_len, HI, d))
    # include extreme codes: +-448 and subnormals
    q[0, 0, :4] = [0x7E, 0xFE, 0x01, 0x81]
    k = _rand_fp8(rng, (B, S, d))
    k[1, 2, :4] = [0x7E, 0x7E, 0x03, 0x85]
    w = encode_bf16_rne((rng.standard_normal((B * q_len, HI)) / 8).astype(np.float32))
    ks = (rng.random((B, S)) * 0.02 + 0.001).astype(np.float32)
    qs = (rng.random((B * q_len, HI)) * 2 + 0.5).astype(np.float32)
    seq_lens = [5, 4]
    I = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", seq_lens, q_len,
                       k_scale=ks, q_scale=qs)
    qf, kf, wf = decode_e4m3fn(q), decode_e4m3fn(k), decode_bf16(w)
    _, pos = query_positions(seq_lens, q_len)
    for t in range(B * q_len):
        b = t // q_len
        for s in range(S):
            if s > pos[t]:
                assert I[t, s] == -np.inf
                continue
            tot = Fraction(0)
            for j in range(HI):
                dot = sum(Fraction(qf[t, j, e]) * Fraction(kf[b, s, e]) for e in range(d))
                tot += Fraction(wf[t, j]) * Fraction(float(qs[t, j])) * max(dot, Fraction(0))
            exact = tot * Fraction(float(ks[b, s]))
            assert abs(Fraction(I[t, s]) - exact) <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


def test_single_head_unit_weight_is_relu_of_matmul():
    """H_I = 1, w = 1: I = ReLU(q k^T) masked -- a plain GEMM."""
    rng = np.random.default_rng(4)
    T, d, S = 6, 16, 6
    q = rng.standard_normal((T, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, S, d)).astype(np.float32)
    w = np.ones((T, 1), np.float32)
    I = indexer_scores(q, "f32", w, "f32", k, "f32", [S], T)
    ref = np.maximum(q[:, 0, :].astype(np.float64) @ k[0].astype(np.float64).T, 0)
    ref[np.triu_indices(T, 1)] = -np.inf
    assert np.allclose(I, ref, rtol=1e-13, atol=0) and np.array_equal(np.isinf(I), np.isinf(ref))


def test_nonnegative_inputs_reduce_to_weighted_mean_query():
    """w, q, k >= 0: ReLU is the identity, so I = (sum_j w_j q_j) . k."""
    rng = np.random.default_rng(5)
    T, HI, d = 4, 5, 12
    q = rng.random((T, HI, d)).astype(np.float32)
    w = rng.random((T, HI)).astype(np.float32)
    k = rng.random((1, 9, d)).astype(np.float32)
    I = indexer_scores(q, "f32", w, "f32", k, "f32", [9], T)
    u = np.einsum("tj,tjd->td", w.astype(np.float64), q.astype(np.float64))
    ref = u @ k[0].astype(np.float64).T
    pos = np.arange(9 - T, 9)
    for t in range(T):
        assert np.allclose(I[t, :pos[t] + 1], ref[t, :pos[t] + 1], rtol=1e-13)
        assert np.all(np.isneginf(I[t, pos[t] + 1:]))


def test_relu_drops_negative_heads_and_signs_follow_w():
    rng = np.random.default_rng(6)
    d = 8
    k = rng.random((1, 3, d)).astype(np.float32)          # k >= 0
    q = -rng.random((1, 4, d)).astype(np.float32)         # every q.k < 0
    w = rng.standard_normal((1, 4)).astype(np.float32)
    I = indexer_scores(q, "f32", w, "f32", k, "f32", [3], 1)
    assert np.array_equal(I[0], np.zeros(3))
    q2 = -q
    I2 = indexer_scores(q2, "f32", -w, "f32", k, "f32", [3], 1)
    I3 = indexer_scores(q2, "f32", w, "f32", k, "f32", [3], 1)
    assert np.allclose(I2, -I3, rtol=1e-14)


def test_scales_are_positively_homogeneous():
    rng = np.random.default_rng(7)
    T, HI, d, S = 3, 4, 16, 7
    q = _rand_fp8(rng, (T, HI, d))
    k = _rand_fp8(rng, (1, S, d))
    w = encode_bf16_rne(rng.standard_normal((T, HI)).astype(np.float32))
    ks = (rng.random((1, S)) + 0.5).astype(np.float32)
    base = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T, k_scale=ks)
    dbl = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T, k_scale=ks * 2)
    fin = np.isfinite(base)
    assert np.array_equal(dbl[fin], 2 * base[fin])
    qs = np.full((T, HI), 4.0, np.float32)
    q4 = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T, k_scale=ks, q_scale=qs)
    assert np.array_equal(q4[fin], 4 * base[fin])
    # k_scale=None means 1
    one = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T,
                         k_scale=np.ones((1, S), np.float32))
    none = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T)
    assert np.array_equal(one, none)


def test_sequences_only_see_their_own_cache_and_causal_prefix():
    rng = np.random.default_rng(8)
    B, q_len, S, HI, d = 3, 2, 10, 4, 8
    seq_lens = [10, 4, 7]
    q = rng.standard_normal((B * q_len, HI, d)).astype(np.float32)
    w = rng.standard_normal((B * q_len, HI)).astype(np.float32)
    k = rng.standard_normal((B, S, d)).astype(np.float32)
    I = indexer_scores(q, "f32", w, "f32", k, "f32", seq_lens, q_len)
    k2 = k.copy()
    k2[1] *= 1000.0                     # poison sequence 1's cache
    k2[0, 9] = 1e6                      # beyond row 0's position (pos 8)
    I2 = indexer_scores(q, "f32", w, "f32", k2, "f32", seq_lens, q_len)
    same = [0, 4, 5]                    # rows of sequences 0 and 2
    assert np.array_equal(I[same][:, :9], I2[same][:, :9])
    _, pos = query_positions(seq_lens, q_len)
    for t in range(B * q_len):
        assert np.all(np.isfinite(I[t, :pos[t] + 1]))
        assert np.all(np.isneginf(I[t, pos[t] + 1:]))


def test_row_subset_equals_full():
    rng = np.random.default_rng(9)
    T, HI, d, S = 20, 4, 8, 20
    q = _rand_fp8(rng, (T, HI, d))
    k = _rand_fp8(rng, (1, S, d))
    w = encode_bf16_rne(rng.standard_normal((T, HI)).astype(np.float32))
    full = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T, chunk=3)
    rows = np.array([19, 0, 7, 7, 13])
    sub = indexer_scores(q, "e4m3fn", w, "bf16", k, "e4m3fn", [S], T, rows=rows)
    assert np.array_equal(sub, full[rows])
