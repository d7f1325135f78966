"""Seeded block tables for paged caches (input generation only).

A paged cache is a pool of fixed-size pages plus a table ``[B, max_pages]``
of page ids, page ``j`` of sequence ``b`` holding tokens ``j*P .. j*P+P-1``.
The tables drawn here model a serving pool after some churn:

* every sequence owns ``max_pages = ceil(S_max / P)`` table slots; the pages
  behind them are drawn without replacement from a shuffled pool, so
  logically adjacent pages are physically scattered;
* a few spare pages are never referenced;
* optionally sequence 1 shares its first ``share_pages`` pages with
  sequence 0 (a common prompt prefix: same page ids, same contents);
* slots past a sequence's last token are never read by the path, so in the
  ``table`` handed to the kernels they hold wild ids (negative, past the
  pool); ``clean`` points them at one junk page instead, which is what the
  test side uses to build and read the pool.

The last pool page is the junk page.
"""

import numpy as np


def make_block_table(seed, B, seq_lens, S_max, page_size, spare_pages=3, share_pages=0):
    """Returns ``(table, clean, num_pages)``: int32 ``[B, max_pages]`` tables
    (``table`` with wild ids in unread slots, ``clean`` with the junk page
    there) and the pool size in pages."""
    rng = np.random.default_rng([seed, 0x9A6E])
    P = int(page_size)
    max_pages = -(-int(S_max) // P)
    used = B * max_pages
    num_pages = used + spare_pages + 1
    junk = num_pages - 1
    clean = rng.permutation(used + spare_pages)[:used].reshape(B, max_pages).astype(np.int32)
    if share_pages and B > 1:
        clean[1, :share_pages] = clean[0, :share_pages]
    table = clean.copy()
    wild = np.array([-7, num_pages, 1 << 30, -(1 << 30)], dtype=np.int64)
    for b in range(B):
        first_unread = -(-int(seq_lens[b]) // P)
        n = max_pages - first_unread
        if n > 0:
            table[b, first_unread:] = rng.choice(wild, n).astype(np.int32)
            clean[b, first_unread:] = junk
    return table, clean, num_pages


def share_prefix(cache, share_pages, page_size):
    """Copy sequence 0's first ``share_pages`` pages of ``cache`` [B, S, ...]
    into sequence 1, so a shared-prefix table describes one consistent cache."""
    if cache is None or share_pages == 0 or cache.shape[0] < 2:
        return cache
    n = min(share_pages * page_size, cache.shape[1])
    cache = cache.copy()
    cache[1, :n] = cache[0, :n]
    return cache
