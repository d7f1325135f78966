"""GPU parity of the MHA-mode prefill (dsa_mha_prefill, through the C ABI)
against the float64 oracle ``oracle.mha_prefill``.

The decompressed keys and values are bf16 tensors, as the output of the bf16
``wkv_b`` Linear is in the pages' MLA forward code block; the oracle rounds
them the same way (``round_bf16=True``) and is exact from there on.
Tolerance: the attention bar of the MQA path (1e-2 absolute, or half a bf16
ulp of the exact value where that is larger); lse within 1e-2.
"""

import numpy as np
import pytest
import torch

from oracle import mha_prefill as oracle_mha
from synth import make_workload
from tests.gpu_util import attention_tolerance, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(out_gpu, lse_gpu, ref, ref_lse):
    tol = attention_tolerance(ref, True)
    err = np.abs(out_gpu - ref)
    print(f"  max |out - oracle| = {err.max():.3g}", flush=True)
    assert np.all(err <= tol), f"max |out - oracle| = {err.max():.3g} (worst excess {(err - tol).max():.3g})"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse_gpu), fin)
    assert np.all(np.abs(lse_gpu[fin] - ref_lse[fin]) <= 1e-2)


CASES = [
    # name, B, q_len, seq_lens, S_max, H
    ("fresh_ragged", 1, 300, [300], 300, 16),            # two query tiles (44-row tail), 5 key tiles
    ("chunked_two_seqs", 2, 130, [500, 130], 512, 32),   # queries at the end of a longer cache
    ("single_queries", 3, 1, [1, 70, 2048], 2048, 16),   # one query per sequence, one key up to 2048
    ("short_seq_in_batch", 2, 64, [64, 40], 64, 16),      # seq 1 shorter than q_len: 24 rows see nothing
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mha_prefill_small(dsa_gpu, case):
    name, B, q_len, seq, S, H = case
    _say(f"[mha] {name}")
    lcl = dsa_gpu
    seq = np.asarray(seq)
    wl = make_workload(name, B, q_len, np.maximum(seq, q_len), S, 2048, H, seed=31)
    q, kv, w = wl.qh(), wl.kv_all(), wl.wkv_b()
    d_seq = torch.from_numpy(seq.astype(np.int32)).cuda()
    geom = lcl.make_geom(B, q_len, S, d_seq)
    out, lse = lcl.mha_prefill(geom, to_dev(q), to_dev(kv), to_dev(w), wl.sm_scale)
    torch.cuda.synchronize()
    got, got_lse = from_dev(out), lse.cpu().numpy()
    pos = np.repeat(seq, q_len) - q_len + np.tile(np.arange(q_len), B)
    live = np.nonzero(pos >= 0)[0]
    if len(live) < B * q_len:   # rows that see no key: zero output, lse = -inf
        dead = np.nonzero(pos < 0)[0]
        assert np.all(got[dead] == 0) and np.all(np.isneginf(got_lse[dead]))
    # the oracle needs q_len <= seq_lens; rows of shorter sequences are checked one by one
    if np.all(seq >= q_len):
        ref, ref_lse = oracle_mha(q, "bf16", kv, "bf16", w, "bf16", seq, q_len, wl.sm_scale, rows=live,
                                  round_bf16=True)
    else:
        ref, ref_lse = _oracle_short(q, kv, w, seq, q_len, wl.sm_scale, live)
    _check(got[live], got_lse[live], ref, ref_lse)


def _oracle_short(q, kv, w, seq, q_len, sm, live):
    """Rows of sequences shorter than q_len: each visible row is the last
    query of a geometry whose q_len fits (same position, same keys)."""
    outs, lses = [], []
    for t in live:
        b, i = divmod(int(t), q_len)
        p = int(seq[b]) - q_len + i
        o, l = oracle_mha(q[t:t + 1], "bf16", kv[b:b + 1], "bf16", w, "bf16", np.array([p + 1]), 1, sm,
                          round_bf16=True)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def test_mha_prefill_full_2k_sampled(dsa_gpu):
    """Four 2048-token prompts (= top-k, so every position is kept), 128
    heads: sampled rows and heads against the oracle."""
    lcl = dsa_gpu
    _say("[mha] full 4 x 2048, 128 heads, sampled")
    B, L, H = 4, 2048, 128
    wl = make_workload("mha2k", B, L, L, L, 2048, H, seed=32)
    rows = np.array([0, 1, 255, 256, 1023, 2047, 3 * L + 5, 3 * L + 1500, 3 * L + 2047])
    heads = np.array([0, 1, 77, 127])
    qs = np.zeros((B * L, H, 192), np.uint16)
    qs[rows] = wl.qh(rows)                       # other rows: zero queries (uniform weights), not checked
    kv, w = wl.kv_all(), wl.wkv_b()
    d_seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    geom = lcl.make_geom(B, L, L, d_seq)
    out, lse = lcl.mha_prefill(geom, to_dev(qs), to_dev(kv), to_dev(w), wl.sm_scale)
    torch.cuda.synchronize()
    got = from_dev(out)[rows][:, heads]
    got_lse = lse.cpu().numpy()[rows][:, heads]
    ref, ref_lse = oracle_mha(qs, "bf16", kv, "bf16", w, "bf16", np.full(B, L), L, wl.sm_scale, rows=rows,
                              heads=heads, round_bf16=True)
    _check(got, got_lse, ref, ref_lse)
