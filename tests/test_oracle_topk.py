"""Pins for the oracle's top-k selection ("详解DSA": ``topk(min(index_topk,
end_pos))``; ties toward the lower index)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import topk_select

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_case.json")


def _brute(scores, pos, k):
    """Repeatedly take the largest remaining score, lowest index first."""
    left = list(range(pos + 1))
    chosen = []
    while left and len(chosen) < k:
        best = left[0]
        for s in left[1:]:
            if scores[s] > scores[best]:
                best = s
        chosen.append(best)
        left.remove(best)
    return sorted(chosen)


def test_hand_case():
    g = json.load(open(GOLDEN))
    scores = [[-np.inf if v == "-inf" else float(v) for v in r] for r in g["scores"]]
    pos = [1, 2]
    for k, key in ((1, "top1"), (2, "top2")):
        for t in range(2):
            idx, tau = topk_select(np.array(scores[t]), pos[t], k)
            assert [i for i in idx if i >= 0] == g[key][t]
            exp_tau = g[key + "_tau"][t]
            assert tau == (-np.inf if exp_tau == "-inf" else exp_tau)


@pytest.mark.parametrize("seed", range(6))
def test_matches_brute_force_with_heavy_ties(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        n = int(rng.integers(1, 60))
        pos = int(rng.integers(0, n))
        k = int(rng.integers(1, 70))
        scores = rng.integers(-3, 4, n).astype(np.float64)   # many exact ties
        scores[pos + 1:] = -np.inf
        idx, tau = topk_select(scores, pos, k)
        want = _brute(scores, pos, k)
        got = [int(i) for i in idx if i >= 0]
        assert got == want
        assert len(idx) == k and np.all(idx[len(want):] == -1)
        if pos + 1 > k:
            assert tau == scores[want].min()


def test_short_rows_keep_every_valid_position():
    s = np.array([5.0, -1e30, 3.0, np.inf * 0 + 1.0, -np.inf])
    idx, tau = topk_select(s, 3, 8)
    assert idx.tolist() == [0, 1, 2, 3, -1, -1, -1, -1] and tau == -np.inf
    idx, _ = topk_select(s, 3, 4)
    assert idx.tolist() == [0, 1, 2, 3]


def test_distinct_scores_match_torch_topk():
    rng = np.random.default_rng(11)
    for n, k in ((1000, 64), (5000, 2048), (3000, 1)):
        s = rng.standard_normal(n)
        idx, tau = topk_select(s, n - 1, k)
        ref = torch.topk(torch.from_numpy(s), k).indices.numpy()
        assert set(idx.tolist()) == set(ref.tolist())
        assert tau == s[ref].min()


def test_k1_is_first_argmax():
    s = np.array([1.0, 7.0, 3.0, 7.0, 7.0])
    idx, tau = topk_select(s, 4, 1)
    assert idx.tolist() == [int(np.argmax(s))] == [1] and tau == 7.0


def test_boundary_group_takes_lowest_indices():
    # ten-way tie at the boundary: 3 larger values, then pick the 2 lowest tied
    s = np.full(20, 0.5)
    s[[4, 9, 17]] = 2.0
    s[[0, 1]] = -1.0
    idx, tau = topk_select(s, 19, 5)
    assert idx.tolist() == [2, 3, 4, 9, 17] and tau == 0.5
