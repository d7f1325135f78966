"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances: indexer scores within 2e-2 relative; top-k sets identical outside
a 1e-3-relative band around the k-th score (and bit-exact when dsa_topk runs on
the GPU's own scores); attention outputs within 1e-2 max-abs.
"""

import numpy as np
import pytest
import torch

from oracle import query_positions, topk_select
from synth import standard_workload, make_workload
from tests.gpu_util import Uploaded, check_attention, check_scores, check_topk, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


SMALL = [
    # name, B, q_len, seq_lens, S_max, topk, H, fp8, ki_mode
    ("decode_ragged", 3, 1, [3000, 1777, 2049], 3000, 256, 32, True, "normal"),
    ("decode_two_q", 4, 2, [5000, 4095, 4097, 300], 5000, 512, 16, True, "normal"),
    ("decode_ties", 2, 2, [6000, 5001], 6000, 256, 16, True, "pool"),
    ("prefill_small", 1, 700, [700], 700, 128, 16, True, "normal"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_indexer_and_topk_small(dsa_gpu, case):
    name, B, q_len, seq, S, k, H, fp8, mode = case
    _say(f"[indexer+topk] {name}")
    wl = make_workload(name, B, q_len, seq, S, k, H, fp8=fp8, seed=11, ki_mode=mode)
    up = Uploaded(wl, with_mla=False)
    g = up.geom(dsa_gpu)
    sc = dsa_gpu.indexer_scores(g, up.d_qi, up.d_w, up.d_ki, k_scale=up.d_ks)
    idx = dsa_gpu.topk(g, sc, k)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    ref = up.oracle_scores()
    pos = wl.positions()
    check_scores(got, ref, pos)
    check_topk(idx.cpu().numpy(), ref, pos, k)
    # standalone top-k on the GPU's own scores must equal the oracle rule bit-exactly
    gi = idx.cpu().numpy()
    for r in range(wl.T):
        want, _ = topk_select(got[r].astype(np.float64), pos[r], k)
        assert np.array_equal(gi[r], want), f"row {r}: dsa_topk differs from the selection rule on its own scores"


def test_indexer_row_slice_and_ld(dsa_gpu):
    _say("[indexer] row slice with padded ld")
    wl = make_workload("slice", 2, 40, [3000, 2500], 3000, 64, 16, seed=12)
    up = Uploaded(wl, with_mla=False)
    g = up.geom(dsa_gpu)
    ld = 3008
    buf = torch.full((30, ld), 7.0, device="cuda")
    dsa_gpu.indexer_scores(g, up.d_qi, up.d_w, up.d_ki, k_scale=up.d_ks, row_begin=25, row_count=30, scores=buf)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    rows = np.arange(25, 55)
    ref = up.oracle_scores(rows=rows)
    check_scores(got[:, :3000], ref, wl.positions()[rows])
    assert np.all(got[:, 3000:] == 7.0), "columns beyond S_max must be untouched"


TOPK_PATHS = [
    # name, S, extra columns (ld = S + extra)
    ("one_block_per_row", 20000, 0),             # 16-byte score loads
    ("one_block_per_row_odd_ld", 30001, 1),      # ld % 4 != 0: 4-byte loads
    ("several_blocks_per_row", 40000, 0),        # rows beyond 32768 scores
]


@pytest.mark.parametrize("case", TOPK_PATHS, ids=[c[0] for c in TOPK_PATHS])
def test_topk_synthetic_ties_and_short_rows(dsa_gpu, case):
    """Rows up to 32768 scores (k <= 2048) are selected by one block each,
    longer rows (or k > 2048) by several; every path must follow the rule
    exactly.  Columns past S_max hold a huge score that must never be read."""
    name, S, extra = case
    _say(f"[topk] synthetic ties / short rows / concentrated rows, {name}")
    rng = np.random.default_rng(5)
    B, q_len = 6, 1
    seq = np.array([S, 17, S, S, 9000, 2049], np.int32)
    scores = np.full((B, S + extra), 1e30, np.float32)
    scores[:, :S] = rng.integers(-5, 6, (B, S))                       # massive ties
    scores[2, :S] = 1.0                                                # one value everywhere
    scores[3, :S] = 1.0 + rng.standard_normal(S) * 1e-6                # all in one bin
    scores[4, :S] = rng.standard_normal(S)
    d_seq = torch.from_numpy(seq).cuda()
    g = dsa_gpu.make_geom(B, q_len, S, d_seq)
    for k in (1, 7, 2048, 4096):
        idx = dsa_gpu.topk(g, torch.from_numpy(scores).cuda(), k).cpu().numpy()
        for r in range(B):
            want, _ = topk_select(scores[r, :S].astype(np.float64), seq[r] - 1, k)
            assert np.array_equal(idx[r], want), f"k={k} row {r}"


MLA_CASES = [
    # name, B, q_len, seq_lens, S_max, k, H, bf16
    ("decode_bf16", 3, 2, [5000, 3000, 2], 5000, 512, 128, True),
    ("decode_bf16_h32", 2, 1, [4000, 100], 4000, 300, 32, True),
    # 96 rows, k = 1024: one split per row, each row's 128 heads as two
    # 64-head blocks that write the output directly (no partials)
    ("decode_bf16_halves_1split", 48, 2, [2500, 1800, 1100, 2500, 2047, 1025] * 8, 2500, 1024, 128, True),
    # one query, 128 heads, top-2048: 8 splits x two 64-head blocks (16 blocks)
    ("decode_bf16_one_query", 1, 1, [3000], 3000, 2048, 128, True),
    ("prefill_bf16", 1, 96, [1000], 1000, 256, 64, True),
    ("tiny_f32", 1, 64, [200], 200, 64, 16, False),
]


def test_topk_largest_rows(dsa_gpu):
    """The largest rows the top-k accepts (S_max = 262144) at k = 2048 and
    the largest k (4096): ragged lengths, a tied row, a row of exactly k + 1
    valid positions; exact against the oracle's rule."""
    _say("[topk] S_max = 262144, k in (2048, 4096)")
    rng = np.random.default_rng(8)
    S = 262144
    seq = np.array([S, 100003, 4097, S], np.int32)
    B = len(seq)
    scores = rng.standard_normal((B, S)).astype(np.float32)
    scores[3] = rng.integers(-3, 4, S)                          # heavy ties over the whole row
    d_seq = torch.from_numpy(seq).cuda()
    g = dsa_gpu.make_geom(B, 1, S, d_seq)
    for k in (2048, 4096):
        idx = dsa_gpu.topk(g, torch.from_numpy(scores).cuda(), k).cpu().numpy()
        for r in range(B):
            want, _ = topk_select(scores[r].astype(np.float64), seq[r] - 1, k)
            assert np.array_equal(idx[r], want), f"k={k} row {r}"


def test_topk_threshold_bin_regimes(dsa_gpu):
    """128K rows (several blocks per row), k = 2048, built so the threshold
    bin's candidates take each branch of the final selection: few
    candidates (at most 4096: four register slots per thread), a crowded
    bin (4096 < candidates <= 2k + 4096: twelve slots) whose next 10 bits are
    resolved by the second histogram with ties at the k-th score, a bin
    whose next 10 bits hold exactly the remaining count (taken whole), and an
    overflowing bin (the selection falls back to the score row).  Further
    rows: 3000 distinct top scores on odd positions only, candidates on both
    sides of zero (the k-th score negative), and infinite scores.  Exact
    against the oracle's rule."""
    _say("[topk] 128K rows: threshold-bin regimes of the final selection")
    S_max = 131076                                       # every row holds 131072 valid scores
    rng = np.random.default_rng(21)
    S, k = 131072, 2048
    B = 7
    scores = np.full((B, S_max), 1e30, np.float32)     # columns past S are never read
    scores[:, :S] = rng.uniform(-1.0, 0.5, (B, S)).astype(np.float32)
    # row 0: a plain spread, few candidates in the threshold bin
    scores[0, :S] = rng.standard_normal(S).astype(np.float32)
    # row 1: 1500 clear winners, then 5000 scores inside [1, 1.125) drawn
    # from 640 values (ties at the k-th score)
    p1 = rng.permutation(S)
    scores[1, p1[:1500]] = rng.uniform(100.0, 200.0, 1500)
    scores[1, p1[1500:6500]] = (1.0 + rng.integers(0, 640, 5000) / 8192.0).astype(np.float32)
    # row 2: 2000 winners, then a digit holding exactly 48 scores
    p2 = rng.permutation(S)
    scores[2, p2[:2000]] = rng.uniform(100.0, 200.0, 2000)
    scores[2, p2[2000:2048]] = np.float32(1.0 + 1023.0 / 8192.0)       # the highest digit of [1, 1.125)
    scores[2, p2[2048:5000]] = (1.0 + rng.integers(0, 1000, 2952) / 8192.0).astype(np.float32)
    # row 3: 9000 scores in one narrow range above everything else
    p3 = rng.permutation(S)
    scores[3, p3[:9000]] = (1.0 + rng.integers(0, 1024, 9000) / 8192.0).astype(np.float32)
    # row 4: 3000 distinct top scores at odd positions only (the range
    # sample reads every 128th position)
    odd = rng.permutation(np.arange(1, S, 2))[:3000]
    scores[4, :S] = rng.uniform(-1.0, 0.0, S).astype(np.float32)
    scores[4, odd] = rng.uniform(10.0, 20.0, 3000).astype(np.float32)
    # row 5: only 1000 positive scores, so the top-k reaches into the negatives
    scores[5, :S] = -rng.uniform(1e-3, 5.0, S).astype(np.float32)
    scores[5, rng.permutation(S)[:1000]] = rng.uniform(1e-3, 5.0, 1000).astype(np.float32)
    # row 6: 40 +inf, 3000 -inf, 10 equal largest finite scores
    p6 = rng.permutation(S)
    scores[6, p6[:40]] = np.inf
    scores[6, p6[40:3040]] = -np.inf
    scores[6, p6[3040:3050]] = 3.0e38
    seq = np.full(B, S, np.int32)
    d_seq = torch.from_numpy(seq).cuda()
    g = dsa_gpu.make_geom(B, 1, S_max, d_seq)
    idx = dsa_gpu.topk(g, torch.from_numpy(scores).cuda(), k).cpu().numpy()
    for r in range(B):
        want, _ = topk_select(scores[r, :S].astype(np.float64), S - 1, k)
        assert np.array_equal(idx[r], want), f"row {r}"


@pytest.mark.parametrize("case", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_sparse_mla(dsa_gpu, case):
    name, B, q_len, seq, S, k, H, bf16 = case
    _say(f"[sparse_mla] {name}")
    wl = make_workload(name, B, q_len, seq, S, k, H, fp8=bf16, seed=13)
    up = Uploaded(wl)
    rng = np.random.default_rng(3)
    pos = wl.positions()
    idx = np.full((wl.T, k), -1, np.int32)
    for t in range(wl.T):
        n = min(k, pos[t] + 1) - (t % 3)  # some rows not full
        if n > 0:
            idx[t, :n] = rng.choice(pos[t] + 1, n, replace=False)
        rng.shuffle(idx[t])
    out, lse = dsa_gpu.sparse_mla(up.geom(dsa_gpu), up.d_qm, up.d_kv, to_dev(idx), wl.sm_scale)
    torch.cuda.synchronize()
    check_attention(from_dev(out), lse.cpu().numpy(), up, idx.astype(np.int64), np.arange(wl.T))


FWD_CASES = [
    ("fwd_decode", 4, 2, [6000, 3001, 4500, 2048], 6000, 512, 32, "normal"),
    ("fwd_decode_ties", 2, 2, [7000, 7000], 7000, 512, 16, "pool"),
    ("fwd_prefill_stream", 1, 1500, [1500], 1500, 256, 16, "normal"),
    ("fwd_prefill_stream_b2", 2, 200, [2600, 300], 2600, 128, 16, "normal"),
    ("fwd_prefill_stream_b5", 5, 96, [700, 300, 1200, 96, 2000], 2000, 256, 16, "normal"),  # rotated sequence order
    # streamed lists of capacity 8192 (k = 4096): compactions on the list in global memory
    ("fwd_prefill_stream_k4096", 1, 96, [9000], 9000, 4096, 16, "normal"),
    # k = 2900: the list capacity held at the 3968-word LDS staging area (1068 entries of headroom)
    ("fwd_prefill_stream_k2900", 1, 128, [7000], 7000, 2900, 16, "normal"),
    ("fwd_keep_all", 2, 70, [300, 100], 300, 512, 16, "normal"),   # S_max <= topk: indexer bypassed
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward(dsa_gpu, case):
    name, B, q_len, seq, S, k, H, mode = case
    _say(f"[forward] {name}")
    wl = make_workload(name, B, q_len, seq, S, k, H, seed=14, ki_mode=mode)
    up = Uploaded(wl)
    g = up.geom(dsa_gpu)
    idx, out, lse = dsa_gpu.forward(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                    index_k_scale=up.d_ks)
    sel = dsa_gpu.indexer_topk(g, k, up.d_qi, up.d_w, up.d_ki, index_k_scale=up.d_ks)
    torch.cuda.synchronize()
    assert torch.equal(sel, idx), "dsa_indexer_topk differs from dsa_forward's selection"
    gi = idx.cpu().numpy()
    ref = up.oracle_scores()
    pos = wl.positions()
    check_topk(gi, ref, pos, k)
    check_attention(from_dev(out), lse.cpu().numpy(), up, gi.astype(np.int64), np.arange(wl.T))


# ---------------------------------------------------------------- full sizes

def test_full_tiny512(dsa_gpu):
    _say("[full] tiny512 (fp32 throughout)")
    wl = standard_workload("tiny512")
    up = Uploaded(wl)
    g = up.geom(dsa_gpu)
    sc = dsa_gpu.indexer_scores(g, up.d_qi, up.d_w, up.d_ki)
    idx, out, lse = dsa_gpu.forward(g, wl.topk, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv)
    torch.cuda.synchronize()
    ref = up.oracle_scores()
    pos = wl.positions()
    check_scores(sc.cpu().numpy(), ref, pos)
    gi = idx.cpu().numpy()
    check_topk(gi, ref, pos, wl.topk)
    check_attention(out.cpu().numpy().astype(np.float64), lse.cpu().numpy(), up, gi.astype(np.int64),
                    np.arange(wl.T))


@pytest.mark.parametrize("name", ["decode32k", "decode128k"])
def test_full_decode(dsa_gpu, name):
    _say(f"[full] {name}")
    wl = standard_workload(name)
    up = Uploaded(wl)
    g = up.geom(dsa_gpu)
    idx, out, lse = dsa_gpu.forward(g, wl.topk, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                    index_k_scale=up.d_ks)
    sel = dsa_gpu.indexer_topk(g, wl.topk, up.d_qi, up.d_w, up.d_ki, index_k_scale=up.d_ks)
    sc = dsa_gpu.indexer_scores(g, up.d_qi, up.d_w, up.d_ki, k_scale=up.d_ks)
    torch.cuda.synchronize()
    assert torch.equal(sel, idx), "dsa_indexer_topk differs from dsa_forward's selection"
    ref = up.oracle_scores()
    pos = wl.positions()
    got = sc.cpu().numpy()
    check_scores(got, ref, pos)
    gi = idx.cpu().numpy()
    check_topk(gi, ref, pos, wl.topk)
    for r in range(wl.T):  # the forward's selection is the rule applied to the GPU's own scores
        want, _ = topk_select(got[r].astype(np.float64), pos[r], wl.topk)
        assert np.array_equal(gi[r], want), f"row {r}"
    check_attention(from_dev(out), lse.cpu().numpy(), up, gi.astype(np.int64), np.arange(wl.T))


def _check_sampled_scores(lcl, up, g, sample):
    """dsa_indexer_scores on the sampled rows (row slices of the ABI, one
    launch per run of consecutive rows) against the oracle: the X12 criterion
    on the very scores the streamed forward never writes out."""
    wl = up.wl
    runs = np.split(sample, np.nonzero(np.diff(sample) != 1)[0] + 1)
    got = np.empty((len(sample), wl.S_max), np.float32)
    r = 0
    for run in runs:
        sc = lcl.indexer_scores(g, up.d_qi, up.d_w, up.d_ki, k_scale=up.d_ks, row_begin=int(run[0]),
                                row_count=len(run))
        torch.cuda.synchronize()
        got[r:r + len(run)] = sc.cpu().numpy()
        r += len(run)
    ref = up.oracle_scores(rows=sample)
    worst = check_scores(got, ref, wl.positions()[sample])
    _say(f"  indexer scores on {len(sample)} sampled rows: worst relative error {worst:.3g}")
    return ref


def test_full_prefill8k_planted(dsa_gpu):
    _say("[full] prefill8k planted (streaming path)")
    wl = standard_workload("prefill8k")
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([wl.planted_rows, [0, 1, 2046, 2047, 2048, 2049, 8191],
                                       rng.choice(8192, 24, replace=False)]))
    up = Uploaded(wl, qm_rows=sample)
    g = up.geom(dsa_gpu)
    idx, out, lse = dsa_gpu.forward(g, wl.topk, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                    index_k_scale=up.d_ks)
    sel = dsa_gpu.indexer_topk(g, wl.topk, up.d_qi, up.d_w, up.d_ki, index_k_scale=up.d_ks)
    torch.cuda.synchronize()
    assert torch.equal(sel, idx), "dsa_indexer_topk differs from dsa_forward's selection"
    gi = idx.cpu().numpy()
    for t in wl.planted_rows:
        assert np.array_equal(gi[t], wl.planted_set), f"planted row {t} lost its planted set"
    ref = _check_sampled_scores(dsa_gpu, up, g, sample)
    check_topk(gi[sample], ref, wl.positions()[sample], wl.topk)
    check_attention(from_dev(out)[sample], lse.cpu().numpy()[sample], up, gi[sample].astype(np.int64), sample)


def test_full_prefill64k_sampled(dsa_gpu):
    """Boundary rows {0, 1, 2, k-2 .. k+1}, the last 64 rows and 256 seeded
    random rows of the 64K prefill: scores (X12), selection and attention."""
    _say("[full] prefill64k sampled rows (streaming path)")
    wl = standard_workload("prefill64k")
    rng = np.random.default_rng(2)
    k = wl.topk
    sample = np.unique(np.concatenate([[0, 1, 2, k - 2, k - 1, k, k + 1], np.arange(65536 - 64, 65536),
                                       rng.choice(65536, 256, replace=False)]))
    up = Uploaded(wl, qm_rows=sample)
    g = up.geom(dsa_gpu)
    idx, out, lse = dsa_gpu.forward(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                    index_k_scale=up.d_ks, want_lse=True)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()[sample]
    ref = _check_sampled_scores(dsa_gpu, up, g, sample)
    check_topk(gi, ref, wl.positions()[sample], k)
    check_attention(from_dev(out[torch.from_numpy(sample).cuda()]), lse.cpu().numpy()[sample], up,
                    gi.astype(np.int64), sample)


def test_forward_without_idx_out(dsa_gpu):
    """idx_out = NULL keeps the selection in the workspace; the attention
    output is bit-identical to the call that returns the selection (decode
    with a materialised score buffer, and a streamed prefill)."""
    for name, B, q_len, seq, S, k, H in (("noidx_decode", 3, 2, [5000, 3001, 4097], 5000, 512, 32),
                                         ("noidx_prefill", 1, 600, [600], 600, 128, 16)):
        _say(f"[forward] {name}: idx_out NULL")
        wl = make_workload(name, B, q_len, seq, S, k, H, seed=15)
        up = Uploaded(wl)
        g = up.geom(dsa_gpu)
        idx, out, lse = dsa_gpu.forward(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                        index_k_scale=up.d_ks)
        none, out2, lse2 = dsa_gpu.forward(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                           index_k_scale=up.d_ks, idx=False)
        torch.cuda.synchronize()
        assert none is None
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)
