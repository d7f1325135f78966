"""Pins for the oracle's paged-cache reading (``oracle.paged``): the block
table maps position s of sequence b to row s % P of page table[b, s // P]."""

import numpy as np
import pytest

from oracle import indexer_scores
from oracle.paged import gather_pages, scatter_pages


def test_identity_table_is_the_contiguous_cache():
    rng = np.random.default_rng(0)
    B, S, P = 2, 256, 64
    cache = rng.integers(0, 255, (B, S, 8)).astype(np.uint8)
    pool = cache.reshape(B * S // P, P, 8)                       # page i = rows [64i, 64i+64) of the flat cache
    table = np.arange(B * S // P).reshape(B, S // P)
    assert np.array_equal(gather_pages(pool, table, S), cache)


def test_position_to_page_and_offset_by_hand():
    P = 4
    pool = np.arange(6 * P).reshape(6, P)                        # pool[p, r] = 4p + r
    table = np.array([[5, 0, 3]])
    got = gather_pages(pool, table, 12)[0]
    # s = 0..3 -> page 5 rows 0..3; s = 4..7 -> page 0; s = 8..11 -> page 3
    assert list(got) == [20, 21, 22, 23, 0, 1, 2, 3, 12, 13, 14, 15]


def test_scatter_then_gather_round_trips_and_scores_are_unchanged():
    rng = np.random.default_rng(1)
    B, q_len, S, P, pages = 2, 2, 512, 64, 40
    seq_lens = np.array([512, 300])
    table = rng.permutation(pages)[:B * S // P].reshape(B, S // P)
    ki = rng.integers(0, 0x7E, (B, S, 128)).astype(np.uint8)
    ks = rng.uniform(0.5, 2, (B, S)).astype(np.float32)
    qi = rng.integers(0, 0x7E, (B * q_len, 64, 128)).astype(np.uint8)
    w = rng.standard_normal((B * q_len, 64)).astype(np.float32)
    kpool, spool = scatter_pages(ki, table, pages, P), scatter_pages(ks, table, pages, P)
    assert np.array_equal(gather_pages(kpool, table, S), ki)
    a = indexer_scores(qi, "e4m3fn", w, "f32", ki, "e4m3fn", seq_lens, q_len, k_scale=ks)
    b = indexer_scores(qi, "e4m3fn", w, "f32", gather_pages(kpool, table, S), "e4m3fn", seq_lens, q_len,
                       k_scale=gather_pages(spool, table, S))
    assert np.array_equal(a, b)


def test_out_of_range_page_rejected():
    with pytest.raises(ValueError):
        gather_pages(np.zeros((2, 4)), np.array([[0, 2]]), 8)
