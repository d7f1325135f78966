"""GPU parity on inputs that drive the kernels' rarely taken branches,
against the float64 oracle (through the C ABI):

* sparse MLA whose later tiles hold logits far above the first tile's
  maximum (more than 64 in log2 units), with one split and with several:
  the bf16 attention fixes its softmax reference at the first tile and must
  rerun the split with the true maximum;
* MHA-mode prefill whose logits keep growing along the keys, plus one key
  far above the rest: the running reference moves past its 2^8 margin;
* the indexer KL objective with large attention logits and index scores
  that rise along the set (the online maximum of I moves at almost every
  entry);
* the streamed long-prefill top-k on keys drawn from a small pool, so
  exact score ties sit at the k-th score of most rows: besides the band
  check, no unselected position may come before a selected one holding the
  same key bytes (the lower-index rule, checked with no band).

Tolerances are the ones of the ordinary cases.
"""

import numpy as np
import pytest
import torch

from oracle import attention_lse, indexer_kl as oracle_kl, mha_prefill as oracle_mha, query_positions
from synth import make_workload
from synth.encode import encode_bf16_rne
from tests.gpu_util import check_attention, check_topk, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _bf16_to_f32(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


class _View:
    """What check_attention reads: the workload, its MLA queries and latent cache."""

    def __init__(self, wl, qm, kv):
        self.wl, self.qm, self.kv = wl, qm, kv


# name, B, q_len, seq_lens, S_max, k (k = 128: one split per row; k = 2048 with
# four rows: eight splits of 256 entries)
RERUN = [
    ("one_split", 2, 2, [3000, 2500], 3000, 128),
    ("eight_splits", 2, 2, [5000, 4100], 5000, 2048),
]


@pytest.mark.parametrize("case", RERUN, ids=[c[0] for c in RERUN])
def test_sparse_mla_late_logits_beyond_the_first_tile(dsa_gpu, case):
    name, B, q_len, seq, S, k = case
    H = 128
    _say(f"[extremes] sparse MLA, logits > first tile max + 64 log2 units, {name}")
    wl = make_workload(name, B, q_len, seq, S, k, H, seed=51)
    qm, kv = wl.qm(), wl.kv_all()
    pos = wl.positions()
    rng = np.random.default_rng(52)
    idx = np.full((wl.T, k), -1, np.int32)
    used = set()
    for t in range(wl.T):
        b = t // q_len
        cand = np.array([s for s in rng.permutation(int(pos[t]) + 1)[:k + 64] if (b, s) not in used])[:k]
        idx[t] = cand
        # Two planted rows per head group in tiles 2 and 3 (entries 64.. of the
        # list; within one split): latent row = 2 q[t, h] + noise, so for head h
        # the logit is about sm * 2 * |q|^2 ~ 83 against ~N(0, 3) elsewhere.
        heads = [(37 * t + 16 * j + 3 * j * j) % H for j in range(8)]
        for j, h in enumerate(heads):
            qh = _bf16_to_f32(qm[t, h]).astype(np.float64)
            for m in (64 + 2 * j, 96 + 2 * j + 1):
                s = int(idx[t, m])
                kv[b, s] = encode_bf16_rne((2.0 * qh + 0.3 * rng.standard_normal(576)).astype(np.float32))
                used.add((b, s))
    view = _View(wl, qm, kv)
    d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
    geom = dsa_gpu.make_geom(B, q_len, S, d_seq)
    out, lse = dsa_gpu.sparse_mla(geom, to_dev(qm), to_dev(kv), to_dev(idx), wl.sm_scale)
    torch.cuda.synchronize()
    check_attention(from_dev(out), lse.cpu().numpy(), view, idx.astype(np.int64), np.arange(wl.T))


def test_mha_prefill_growing_logits(dsa_gpu):
    """The rope part of key s is scaled by 1 + s/64 (it enters the logits,
    not the values), so logits spread over tens of nats and keep rising with
    s; key 1700 additionally carries 40 q_pe of query 1900, head 5 (a logit
    of about 185 nats for that head)."""
    _say("[extremes] MHA-mode prefill, growing logits")
    lcl = dsa_gpu
    B, L, H = 1, 2048, 16
    wl = make_workload("mha_grow", B, L, L, L, 2048, H, seed=53)
    q, kv, w = wl.qh(), wl.kv_all(), wl.wkv_b()
    s = np.arange(L, dtype=np.float32)
    rope = _bf16_to_f32(kv[0, :, 512:]) * (1.0 + s / 64.0)[:, None]
    kv[0, :, 512:] = encode_bf16_rne(rope.astype(np.float32))
    kv[0, 1700, 512:] = encode_bf16_rne((40.0 * _bf16_to_f32(q[1900, 5, 128:])).astype(np.float32))
    d_seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    geom = lcl.make_geom(B, L, L, d_seq)
    out, lse = lcl.mha_prefill(geom, to_dev(q), to_dev(kv), to_dev(w), wl.sm_scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 300, 1000, 1699, 1700, 1899, 1900, 1901, 2047])
    got, got_lse = from_dev(out)[rows], lse.cpu().numpy()[rows]
    ref, ref_lse = oracle_mha(q, "bf16", kv, "bf16", w, "bf16", np.array([L]), L, wl.sm_scale, rows=rows,
                              round_bf16=True)
    spread = ref_lse.max() - ref_lse.min()
    _say(f"  oracle lse spread over the checked rows: {spread:.1f} nats")
    tol = np.maximum(1e-2, 0.5 * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7))
    err = np.abs(got - ref)
    _say(f"  max |out - oracle| = {err.max():.3g}")
    assert np.all(err <= tol), f"max error {err.max():.3g}"
    assert np.all(np.abs(got_lse - ref_lse) <= 1e-2), f"lse error {np.abs(got_lse - ref_lse).max():.3g}"


def test_kl_large_logits_and_rising_index_scores(dsa_gpu):
    """Attention logits three times the usual scale (lse from the oracle, so
    the head weights stay <= 1) and index scores I = s/4 + 0.1 N(0, 4) that
    rise along the ascending sets, so the online maximum of I moves at almost
    every entry."""
    _say("[extremes] KL objective, large logits, rising index scores")
    lcl = dsa_gpu
    B, q_len, S, H, k = 2, 2, 6000, 128, 1024
    wl = make_workload("kl_big", B, q_len, [6000, 4500], S, k, H, seed=54)
    qm = encode_bf16_rne(3.0 * _bf16_to_f32(wl.qm()))
    kv = wl.kv_all()
    sc = (0.1 * wl.kl_scores() + np.arange(S, dtype=np.float32)[None, :] / 4.0).astype(np.float32)
    _, pos = query_positions(wl.seq_lens, q_len)
    rng = np.random.default_rng(55)
    idx = np.full((wl.T, k), -1, np.int32)
    for t in range(wl.T):
        idx[t] = np.sort(rng.choice(int(pos[t]) + 1, k, replace=False))
    lse = attention_lse(qm, "bf16", kv, "bf16", idx, wl.seq_lens, q_len, wl.sm_scale).astype(np.float32)
    want, want_loss = oracle_kl(qm, "bf16", kv, "bf16", lse, sc, idx, wl.seq_lens, q_len, wl.sm_scale)
    d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
    geom = lcl.make_geom(B, q_len, S, d_seq)
    kl, loss = lcl.indexer_kl(geom, to_dev(qm), to_dev(kv), to_dev(lse), to_dev(sc), wl.sm_scale, idx=to_dev(idx))
    torch.cuda.synchronize()
    got = kl.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    _say(f"  max |kl - oracle| = {err.max():.3g} (oracle kl in [{want.min():.3g}, {want.max():.3g}])")
    assert np.all(err <= 2e-4 + 1e-4 * np.abs(want)), f"max error {err.max():.3g}"
    assert abs(float(loss.item()) - want_loss) <= 1e-4 * abs(want_loss) + 2e-4


def _key_groups(ki, ks):
    """Group id of every cache position: positions with identical key codes
    and scale bytes share a group (their scores are equal for any query)."""
    B, S, _ = ki.shape
    raw = np.concatenate([ki.reshape(B * S, -1), ks.reshape(B * S).view(np.uint8).reshape(B * S, 4)], axis=1)
    _, inv = np.unique(np.ascontiguousarray(raw).view(np.dtype((np.void, raw.shape[1]))).ravel(),
                       return_inverse=True)
    return inv.reshape(B, S)


STREAM_TIES = [
    # name, B, q_len, seq_lens, S_max, topk, H
    ("pool_one_seq", 1, 1500, [1500], 1500, 256, 16),
    ("pool_two_seqs", 2, 200, [2600, 300], 2600, 128, 16),
    ("pool_k2048", 1, 4096, [4096], 4096, 2048, 16),
]


@pytest.mark.parametrize("case", STREAM_TIES, ids=[c[0] for c in STREAM_TIES])
def test_streamed_prefill_ties_go_to_the_lower_position(dsa_gpu, case):
    name, B, q_len, seq, S, k, H = case
    _say(f"[extremes] streamed prefill top-k on pooled keys (exact ties), {name}")
    wl = make_workload(name, B, q_len, seq, S, k, H, seed=56, ki_mode="pool")
    qi, w = wl.qi(), wl.w()
    ki, ks = wl.ki_all()
    qm, kv = wl.qm(), wl.kv_all()
    d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
    geom = dsa_gpu.make_geom(B, q_len, S, d_seq)
    idx, out, lse = dsa_gpu.forward(geom, k, wl.sm_scale, to_dev(qi), to_dev(w), to_dev(ki), to_dev(qm),
                                    to_dev(kv), index_k_scale=to_dev(ks))
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    pos = wl.positions()
    from oracle import indexer_scores
    ref = indexer_scores(qi, "e4m3fn", w, "bf16", ki, "e4m3fn", wl.seq_lens, q_len, k_scale=ks)
    check_topk(gi, ref, pos, k)
    groups = _key_groups(ki, ks)
    tied_rows = 0
    for t in range(wl.T):
        b, p = t // q_len, int(pos[t])
        if p + 1 <= k:
            continue
        sel = np.zeros(p + 1, bool)
        sel[gi[t][gi[t] >= 0]] = True
        g = groups[b, :p + 1]
        # per group: the selected positions must be the lowest ones of the group
        order = np.lexsort((np.arange(p + 1), g))
        gs, ss = g[order], sel[order]
        starts = np.r_[0, np.nonzero(np.diff(gs))[0] + 1]
        n_sel = np.add.reduceat(ss.astype(np.int64), starts)
        sizes = np.diff(np.r_[starts, len(gs)])
        rank = np.arange(len(gs)) - np.repeat(starts, sizes)
        want = rank < np.repeat(n_sel, sizes)
        assert np.array_equal(ss, want), f"row {t}: a selected position comes after an unselected equal key"
        tied_rows += int(np.any((n_sel > 0) & (n_sel < sizes)))
    _say(f"  rows whose selection cuts a group of equal keys: {tied_rows} of {wl.T}")
    assert tied_rows > 0
    rows = np.arange(wl.T) if wl.T <= 1500 else np.unique(np.r_[np.arange(0, wl.T, 37), wl.T - 1])
    check_attention(from_dev(out)[rows], lse.cpu().numpy()[rows], _View(wl, qm, kv), gi[rows].astype(np.int64),
                    rows)
