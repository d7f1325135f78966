"""GPU parity of the paged-cache entry points (dsa_indexer_scores_paged,
dsa_sparse_mla_paged, dsa_forward_paged, dsa_indexer_cache_append_paged,
through the C ABI).

The oracle reads a paged cache as the contiguous cache its table describes
(``oracle.gather_pages``) and then applies the unchanged definitions, so the
tolerances are those of the contiguous path.  On top of that, a paged call
must reproduce the contiguous call on that same cache bit for bit: the
kernels do the same arithmetic in the same order, only the addresses differ.

Tables come from ``synth.make_block_table``: scattered pages, spare pages,
an optional shared prefix, and wild ids in the slots past each sequence's
last token (the path never reads them).
"""

import numpy as np
import pytest
import torch

from oracle import cache_append, gather_pages, indexer_scores, scatter_pages
from synth import make_block_table, make_workload, share_prefix, standard_workload
from tests.gpu_util import check_attention, check_scores, check_topk, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


class _OracleView:
    """What check_attention reads: the workload, its MLA queries and the
    contiguous latent cache the table describes."""

    def __init__(self, wl, qm, kv):
        self.wl, self.qm, self.kv = wl, qm, kv


class PagedCase:
    """A workload's caches laid out in page pools (host copies for the oracle,
    device copies for the kernels), and the contiguous view of them."""

    def __init__(self, lcl, wl, page_size, seed, share_pages=0, with_mla=True):
        self.wl, self.P = wl, page_size
        table, clean, num_pages = make_block_table(seed, wl.B, wl.seq_lens, wl.S_max, page_size,
                                                   share_pages=share_pages)
        self.num_pages = num_pages
        ki, ks = wl.ki_all()
        ki, ks = share_prefix(ki, share_pages, page_size), share_prefix(ks, share_pages, page_size)
        self.qi, self.w = wl.qi(), wl.w()
        pool = lambda c: None if c is None else scatter_pages(c, clean, num_pages, page_size)
        view = lambda p: None if p is None else gather_pages(p, clean, wl.S_max)
        self.ki_pool, self.ks_pool = pool(ki), pool(ks)
        self.ki, self.ks = view(self.ki_pool), view(self.ks_pool)        # what the oracle reads
        self.d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
        self.d_table = torch.from_numpy(table).cuda()
        self.pages = lcl.make_pages(self.d_table, page_size, num_pages)
        self.geom = lcl.make_geom(wl.B, wl.q_len, wl.S_max, self.d_seq)
        self.d_qi, self.d_w = to_dev(self.qi), to_dev(self.w)
        self.d_ki_pool, self.d_ks_pool = to_dev(self.ki_pool), to_dev(self.ks_pool)
        self.d_ki, self.d_ks = to_dev(self.ki), to_dev(self.ks)          # contiguous twin
        if with_mla:
            self.qm = wl.qm()
            kv = share_prefix(wl.kv_all(), share_pages, page_size)
            self.kv_pool = pool(kv)
            self.kv = view(self.kv_pool)
            self.d_qm, self.d_kv_pool, self.d_kv = to_dev(self.qm), to_dev(self.kv_pool), to_dev(self.kv)
            self.view = _OracleView(wl, self.qm, self.kv)

    def oracle_scores(self):
        wl = self.wl
        return indexer_scores(self.qi, wl.qi_fmt, self.w, wl.w_fmt, self.ki, wl.ki_fmt, wl.seq_lens, wl.q_len,
                              k_scale=self.ks)


def _same(a, b):
    """Bit equality of two device tensors."""
    a, b = a.contiguous(), b.contiguous()
    return a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


PAGED = [
    # name, B, q_len, seq_lens, S_max, topk, H, page_size, fp8, ki_mode, share_pages
    ("p64_ragged", 4, 1, [3000, 64, 1777, 129], 3000, 256, 32, 64, True, "normal", 0),
    ("p256_two_q_shared", 3, 2, [5000, 4097, 2], 5000, 512, 16, 256, True, "normal", 8),
    ("p8192_ties", 2, 2, [9000, 8193], 9000, 256, 16, 8192, True, "pool", 0),
    ("p128_long_q", 1, 300, [700], 700, 128, 16, 128, True, "normal", 0),       # streamed prefill
    ("p64_stream_two_seqs", 2, 600, [2600, 900], 2600, 256, 16, 64, True, "pool", 4),  # streamed, shared prefix
    ("p64_f32", 2, 20, [512, 100], 512, 64, 16, 64, False, "normal", 1),
    ("p64_keep_all", 2, 40, [300, 41], 300, 512, 16, 64, True, "normal", 0),   # S_max <= topk: indexer bypassed
    ("p64_long_and_short", 2, 1, [40000, 100], 40000, 256, 16, 64, True, "normal", 0),  # multi-launch top-k
]


@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_paged_forward(dsa_gpu, case):
    name, B, q_len, seq, S, k, H, P, fp8, mode, share = case
    _say(f"[paged] {name}: indexer, forward, contiguous twins")
    lcl = dsa_gpu
    wl = make_workload(name, B, q_len, seq, S, k, H, fp8=fp8, seed=21, ki_mode=mode)
    pc = PagedCase(lcl, wl, P, seed=5, share_pages=share)
    sc_p = lcl.indexer_scores(pc.geom, pc.d_qi, pc.d_w, pc.d_ki_pool, k_scale=pc.d_ks_pool, pages=pc.pages)
    sc_c = lcl.indexer_scores(pc.geom, pc.d_qi, pc.d_w, pc.d_ki, k_scale=pc.d_ks)
    idx_p, out_p, lse_p = lcl.forward(pc.geom, k, wl.sm_scale, pc.d_qi, pc.d_w, pc.d_ki_pool, pc.d_qm,
                                      pc.d_kv_pool, index_k_scale=pc.d_ks_pool, pages=pc.pages)
    idx_c, out_c, lse_c = lcl.forward(pc.geom, k, wl.sm_scale, pc.d_qi, pc.d_w, pc.d_ki, pc.d_qm, pc.d_kv,
                                      index_k_scale=pc.d_ks)
    torch.cuda.synchronize()
    ref = pc.oracle_scores()
    pos = wl.positions()
    check_scores(sc_p.cpu().numpy(), ref, pos)
    gi = idx_p.cpu().numpy()
    check_topk(gi, ref, pos, k)
    check_attention(from_dev(out_p), lse_p.cpu().numpy(), pc.view, gi.astype(np.int64), np.arange(wl.T))
    assert _same(sc_p, sc_c), "paged indexer scores differ from the contiguous call"
    assert _same(idx_p, idx_c), "paged selection differs from the contiguous forward"
    assert _same(out_p, out_c) and _same(lse_p, lse_c), "paged attention differs from the contiguous forward"


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_paged_sparse_mla(dsa_gpu, bf16):
    """Index sets with -1, negative and past-position entries (skipped)."""
    lcl = dsa_gpu
    _say(f"[paged] dsa_sparse_mla_paged bf16={bf16}")
    wl = make_workload("pmla", 3, 2, [4000, 65, 2500], 4000, 512, 32, fp8=bf16, seed=22)
    pc = PagedCase(lcl, wl, 64, seed=6)
    rng = np.random.default_rng(7)
    pos = wl.positions()
    idx = np.full((wl.T, 512), -1, np.int32)
    for t in range(wl.T):
        n = min(512 - 4, pos[t] + 1) - (t % 2) * 7               # room for the invalid entries
        idx[t, :n] = rng.choice(pos[t] + 1, n, replace=False)
        idx[t, n:n + 3] = [pos[t] + 1, -5, wl.S_max + 9]        # invalid: skipped
        rng.shuffle(idx[t])
    d_idx = to_dev(idx)
    out_p, lse_p = lcl.sparse_mla(pc.geom, pc.d_qm, pc.d_kv_pool, d_idx, wl.sm_scale, pages=pc.pages)
    out_c, lse_c = lcl.sparse_mla(pc.geom, pc.d_qm, pc.d_kv, d_idx, wl.sm_scale)
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx <= pos[:, None])                  # the oracle takes the valid set only
    check_attention(from_dev(out_p), lse_p.cpu().numpy(), pc.view, np.where(valid, idx, -1).astype(np.int64),
                    np.arange(wl.T))
    assert _same(out_p, out_c) and _same(lse_p, lse_c)


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_paged_cache_append(dsa_gpu, bf16):
    """New keys land in their pages (bit-exact against the oracle's append on
    the contiguous view); every other pool row, spare and junk pages
    included, is untouched."""
    lcl = dsa_gpu
    _say(f"[paged] dsa_indexer_cache_append_paged bf16={bf16}")
    B, q_len, S, P = 4, 3, 1000, 64
    seq = np.array([1000, 3, 130, 64], np.int32)
    table, clean, num_pages = make_block_table(8, B, seq, S, P, share_pages=0)
    rng = np.random.default_rng(9)
    pool_c = rng.integers(0, 256, (num_pages, P, 128), dtype=np.uint8)
    pool_s = rng.standard_normal((num_pages, P)).astype(np.float32)
    x = rng.standard_normal((B, q_len, 128)).astype(np.float32) * 3
    if bf16:
        from synth import encode_bf16_rne
        bits = encode_bf16_rne(x)
        x_dev, x32 = to_dev(bits), (bits.astype(np.uint32) << 16).view(np.float32)
    else:
        x_dev, x32 = to_dev(x), x
    d_seq = torch.from_numpy(seq).cuda()
    d_table = torch.from_numpy(table).cuda()
    d_c, d_s = to_dev(pool_c), to_dev(pool_s)
    geom = lcl.make_geom(B, q_len, S, d_seq)
    lcl.indexer_cache_append(geom, x_dev, d_c, d_s, pages=lcl.make_pages(d_table, P, num_pages))
    torch.cuda.synchronize()
    want_c, want_s = pool_c.copy(), pool_s.copy()
    vc, vs = cache_append(gather_pages(pool_c, clean, S), gather_pages(pool_s, clean, S), x32, seq, q_len)
    for b in range(B):
        for s in range(seq[b] - q_len, seq[b]):
            if s >= 0:
                want_c[clean[b, s // P], s % P] = vc[b, s]
                want_s[clean[b, s // P], s % P] = vs[b, s]
    assert np.array_equal(d_c.cpu().numpy(), want_c)
    assert np.array_equal(d_s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


def test_full_decode128k_paged(dsa_gpu):
    """The 128K decode (16 x 2 queries, top-2048, 128 heads) on 64-token
    pages: bit-exact against the contiguous forward on the same cache, and
    the oracle's verdict on sampled rows."""
    lcl = dsa_gpu
    _say("[paged] full decode128k, 64-token pages")
    wl = standard_workload("decode128k")
    P = 64
    table, clean, num_pages = make_block_table(10, wl.B, wl.seq_lens, wl.S_max, P)
    ki, ks = wl.ki_all()
    kv = wl.kv_all()
    d_ki, d_ks, d_kv = to_dev(ki), to_dev(ks), to_dev(kv)
    # pools on the device: pool page clean[b, j] holds tokens j*P.. of sequence b
    dst = torch.from_numpy(clean.reshape(-1).astype(np.int64)).cuda()
    mk = lambda c, tail: torch.zeros((num_pages, P) + tail, dtype=c.dtype, device="cuda").index_copy_(
        0, dst, c.reshape((-1, P) + tail))
    ki_pool, ks_pool, kv_pool = mk(d_ki, (128,)), mk(d_ks, ()), mk(d_kv, (576,))
    d_seq = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
    d_table = torch.from_numpy(table).cuda()
    geom = lcl.make_geom(wl.B, wl.q_len, wl.S_max, d_seq)
    pages = lcl.make_pages(d_table, P, num_pages)
    qi, w, qm = wl.qi(), wl.w(), wl.qm()
    d_qi, d_w, d_qm = to_dev(qi), to_dev(w), to_dev(qm)
    idx_p, out_p, lse_p = lcl.forward(geom, wl.topk, wl.sm_scale, d_qi, d_w, ki_pool, d_qm, kv_pool,
                                      index_k_scale=ks_pool, pages=pages)
    idx_c, out_c, lse_c = lcl.forward(geom, wl.topk, wl.sm_scale, d_qi, d_w, d_ki, d_qm, d_kv, index_k_scale=d_ks)
    torch.cuda.synchronize()
    assert _same(idx_p, idx_c) and _same(out_p, out_c) and _same(lse_p, lse_c)
    rows = np.array([0, 1, 17, 30])
    ref = indexer_scores(qi, wl.qi_fmt, w, wl.w_fmt, ki, wl.ki_fmt, wl.seq_lens, wl.q_len, k_scale=ks, rows=rows)
    gi = idx_p.cpu().numpy()
    check_topk(gi[rows], ref, wl.positions()[rows], wl.topk)
    check_attention(from_dev(out_p)[rows], lse_p.cpu().numpy()[rows], _OracleView(wl, qm, kv),
                    gi[rows].astype(np.int64), rows)


def _pools(lcl, clean, num_pages, P, caches):
    """Device page pools holding the contiguous device caches [B, S, ...] at
    the pages of ``clean`` (pool page clean[b, j] = tokens j*P.. of sequence b)."""
    dst = torch.from_numpy(clean.reshape(-1).astype(np.int64)).cuda()
    out = []
    for c in caches:
        tail = tuple(c.shape[2:])
        out.append(torch.zeros((num_pages, P) + tail, dtype=c.dtype, device="cuda").index_copy_(
            0, dst, c.reshape((-1, P) + tail)))
    return out


@pytest.mark.parametrize("name", ["prefill8k", "prefill64k"])
def test_full_prefill_paged_streamed(dsa_gpu, name):
    """The 8K (planted) and 64K prefills on 64-token pages stream their scores
    like the contiguous forward (no T x S buffer in the paged workspace):
    selection and attention bit-exact against the contiguous forward on the
    same cache, the planted sets recovered, and the oracle's verdict on
    sampled rows."""
    lcl = dsa_gpu
    _say(f"[paged] full {name}, 64-token pages, streamed")
    wl = standard_workload(name)
    L, k, P = wl.T, wl.topk, 64
    rng = np.random.default_rng(12)
    sample = np.unique(np.r_[[0, 1, k - 1, k, k + 1, L - 1], rng.choice(L, 10, replace=False)])
    if wl.planted_rows is not None:
        sample = np.unique(np.r_[sample, wl.planted_rows[:4]])
    from tests.gpu_util import Uploaded
    up = Uploaded(wl, qm_rows=sample)
    table, clean, num_pages = make_block_table(14, wl.B, wl.seq_lens, wl.S_max, P)
    ki_pool, ks_pool, kv_pool = _pools(lcl, clean, num_pages, P, (up.d_ki, up.d_ks, up.d_kv))
    d_table = torch.from_numpy(table).cuda()
    pages = lcl.make_pages(d_table, P, num_pages)
    g = up.geom(lcl)
    need_p = lcl.forward_paged_workspace_size(wl.B, L, wl.S_max, wl.H, k, lcl.FP8_E4M3FN, lcl.BF16)
    need_c = lcl.forward_workspace_size(wl.B, L, wl.S_max, wl.H, k, lcl.FP8_E4M3FN, lcl.BF16)
    assert need_p == need_c + (L * k * 4 + 255) // 256 * 256       # streamed: no score buffer
    idx_p, out_p, lse_p = lcl.forward(g, k, wl.sm_scale, up.d_qi, up.d_w, ki_pool, up.d_qm, kv_pool,
                                      index_k_scale=ks_pool, pages=pages)
    idx_c, out_c, lse_c = lcl.forward(g, k, wl.sm_scale, up.d_qi, up.d_w, up.d_ki, up.d_qm, up.d_kv,
                                      index_k_scale=up.d_ks)
    torch.cuda.synchronize()
    assert _same(idx_p, idx_c), "paged selection differs from the contiguous forward"
    assert _same(out_p, out_c) and _same(lse_p, lse_c), "paged attention differs from the contiguous forward"
    gi = idx_p.cpu().numpy()
    if wl.planted_rows is not None:
        for t in wl.planted_rows:
            assert np.array_equal(gi[t], wl.planted_set), f"planted row {t} lost its planted set"
    ref = up.oracle_scores(rows=sample)
    check_topk(gi[sample], ref, wl.positions()[sample], k)
    check_attention(from_dev(out_p[torch.from_numpy(sample).cuda()]), lse_p.cpu().numpy()[sample], up,
                    gi[sample].astype(np.int64), sample)
