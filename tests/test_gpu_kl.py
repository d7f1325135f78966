"""GPU parity of the indexer KL objective (dsa_indexer_kl, through the C ABI)
against the float64 oracle ``oracle.indexer_kl``.

Tolerance, from the arithmetic: each row's KL is A/V - log V - C/V + lse_I
with terms of a few tens (fp32: ~1e-6 each), formed from fp32 exponentials
of fp32-accumulated dot products of bf16 inputs (relative error ~1e-6 in
each exponent) and fp32 sums over up to 32K positions (~1e-5 relative at
worst for random-sign rounding); the bound is
|kl_gpu - kl_oracle| <= 2e-4 + 1e-4 |kl_oracle| per row, and 1e-4 relative
on the summed loss.
"""

import numpy as np
import pytest
import torch

from oracle import attention_lse, indexer_kl as oracle_kl, query_positions, topk_select
from synth import make_workload, standard_workload
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(got, want):
    err = np.abs(got - want)
    print(f"  max |kl - oracle| = {err.max():.3g} (oracle kl in [{want.min():.3g}, {want.max():.3g}])", flush=True)
    assert np.all(err <= 2e-4 + 1e-4 * np.abs(want)), f"max error {err.max():.3g}"


def _sets(scores, pos, k):
    """Selected sets S_t = top-k of the scores (ascending, -1 padded)."""
    idx = np.full((len(pos), k), -1, np.int32)
    for t in range(len(pos)):
        sel, _ = topk_select(scores[t].astype(np.float64), pos[t], k)
        idx[t] = sel
    return idx


CASES = [
    # name, B, q_len, seq_lens, S_max, H, k (0: dense, Eq.(5))
    ("dense_ragged", 3, 2, [700, 65, 2], 700, 32, 0),
    ("sparse_k256", 2, 3, [3000, 180], 3000, 64, 256),      # the second sequence keeps every position
    ("sparse_h128", 2, 1, [5000, 4097], 5000, 128, 512),
    ("dense_h128_one_row", 1, 1, [1500], 1500, 128, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kl_small(dsa_gpu, case):
    name, B, q_len, seq, S, H, k = case
    _say(f"[kl] {name}")
    lcl = dsa_gpu
    wl = make_workload(name, B, q_len, seq, S, max(k, 1), H, seed=41)
    qm, kv, sc = wl.qm(), wl.kv_all(), wl.kl_scores()
    _, pos = query_positions(wl.seq_lens, q_len)
    idx = _sets(sc, pos, k) if k else None
    lse = attention_lse(qm, "bf16", kv, "bf16", idx, wl.seq_lens, q_len, wl.sm_scale)
    lse[::2] += np.random.default_rng(5).standard_normal((lse[::2].shape)) * 0.3   # any per-head constant is valid
    lse = lse.astype(np.float32)
    want, want_loss = oracle_kl(qm, "bf16", kv, "bf16", lse, sc, idx, wl.seq_lens, q_len, wl.sm_scale)
    d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
    geom = lcl.make_geom(B, q_len, S, d_seq)
    kl, loss = lcl.indexer_kl(geom, to_dev(qm), to_dev(kv), to_dev(lse), to_dev(sc), wl.sm_scale,
                              idx=None if idx is None else to_dev(idx))
    torch.cuda.synchronize()
    _check(kl.cpu().numpy().astype(np.float64), want)
    assert abs(float(loss.item()) - want_loss) <= 1e-4 * abs(want_loss) + 2e-4


def test_kl_sparse_decode128k_and_dense_decode32k_sampled(dsa_gpu):
    """The 128K decode shape (32 rows, top-2048 sets of the scores, 128
    heads) on every row, and the dense objective over 32K positions on
    sampled rows (the kernel runs every row)."""
    lcl = dsa_gpu
    rng = np.random.default_rng(6)
    for name, k, rows in (("decode128k", 2048, None), ("decode32k", 0, np.array([0, 33, 63]))):
        _say(f"[kl] full {name} {'sparse' if k else 'dense'}")
        wl = standard_workload(name)
        qm, kv, sc = wl.qm(), wl.kv_all(), wl.kl_scores()
        _, pos = query_positions(wl.seq_lens, wl.q_len)
        idx = _sets(sc, pos, k) if k else None
        lse = (5.0 + rng.standard_normal((wl.T, wl.H))).astype(np.float32)
        d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
        geom = lcl.make_geom(wl.B, wl.q_len, wl.S_max, d_seq)
        kl, loss = lcl.indexer_kl(geom, to_dev(qm), to_dev(kv), to_dev(lse), to_dev(sc), wl.sm_scale,
                                  idx=None if idx is None else to_dev(idx))
        torch.cuda.synchronize()
        want, _ = oracle_kl(qm, "bf16", kv, "bf16", lse, sc, idx, wl.seq_lens, wl.q_len, wl.sm_scale, rows=rows)
        got = kl.cpu().numpy().astype(np.float64)
        _check(got if rows is None else got[rows], want)
        assert abs(float(loss.item()) - got.sum()) <= 1e-5 * abs(got.sum()) + 1e-5
