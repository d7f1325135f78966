"""Paged key / latent caches (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The charlestar page ("DeepSeek V3.2 稀疏注意力：Lightning Indexer 与 Top-k
选择") raises paged caches twice: in "Prefill 与 decode 中发生了什么"
(Decode), the mapping of top-k positions to physical KV pages and selected
positions spread over many pages eating the bandwidth saving; and in "Top-k
是算法与 kernel 的交界面", how a logical position becomes a block and an
offset under paged KV (with a paged indexer-logit kernel among the
components it lists).  A paged cache here
is a pool of fixed-size pages plus a block table: token ``s`` of sequence
``b`` lives in row ``s % P`` of page ``block_table[b, s // P]`` (``P`` tokens
per page).  The computation is the same as on a contiguous cache, so the
oracle reads a paged cache by assembling the contiguous one and then applies
the unchanged definitions of ``oracle.dsa``.
"""

import numpy as np


def gather_pages(pool, block_table, S_max):
    """Contiguous ``[B, S_max, ...]`` view of a paged cache.

    ``pool`` [num_pages, P, ...], ``block_table`` [B, max_pages] int page ids.
    Position ``s`` of sequence ``b`` is ``pool[block_table[b, s // P], s % P]``
    for ``s < min(S_max, max_pages * P)``; positions past the table are zero.
    """
    pool = np.asarray(pool)
    table = np.asarray(block_table, dtype=np.int64)
    num_pages, P = pool.shape[:2]
    B, max_pages = table.shape
    if np.any((table < 0) | (table >= num_pages)):
        raise ValueError("page id out of range")
    out = np.zeros((B, S_max) + pool.shape[2:], dtype=pool.dtype)
    n = min(S_max, max_pages * P)
    s = np.arange(n)
    for b in range(B):
        out[b, :n] = pool[table[b, s // P], s % P]
    return out


def scatter_pages(cache, block_table, num_pages, P):
    """Inverse of ``gather_pages`` for building test inputs: a pool holding the
    contiguous ``cache`` [B, S_max, ...] at the pages of ``block_table``
    (unreferenced pages are zero)."""
    cache = np.asarray(cache)
    table = np.asarray(block_table, dtype=np.int64)
    B, S_max = cache.shape[:2]
    pool = np.zeros((num_pages, P) + cache.shape[2:], dtype=cache.dtype)
    n = min(S_max, table.shape[1] * P)
    s = np.arange(n)
    for b in range(B):
        pool[table[b, s // P], s % P] = cache[b, :n]
    return pool
