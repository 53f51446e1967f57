"""Paged KV cache append, written as its plain definition (TEST INFRASTRUCTURE
ONLY: called from the tests and the benchmark, never from the library).

Inference kernel cookbook page, recipe 02 (store each token's K and V once for
later decode steps) and recipe 03 (fixed-size pages reached through a page
table): the token at logical position t of sequence s lives in page
page_table[s][t // page], row t % page, of a [num_pages, H_kv, page, d] pool.
"""
from __future__ import annotations

import numpy as np


def kv_append(k_pool, v_pool, page_table, seq_ids, positions, k_new, v_new, page_size=16):
    """Scatter the rows of new tokens into host pools, in place.

    k_pool, v_pool: uint16 [num_pages, H_kv, page_size, d]; page_table: int32
    [S, max_pages]; seq_ids, positions: int [T]; k_new, v_new: uint16
    [T, H_kv, d].  A token whose sequence, position or page is out of range
    is skipped, as the library's contract states.  Returns the number written.
    """
    S, max_pages = page_table.shape
    num_pages = k_pool.shape[0]
    written = 0
    for i in range(len(seq_ids)):
        s, t = int(seq_ids[i]), int(positions[i])
        if not (0 <= s < S and 0 <= t < max_pages * page_size):
            continue
        page = int(page_table[s, t // page_size])
        if not (0 <= page < num_pages):
            continue
        k_pool[page, :, t % page_size, :] = k_new[i]
        v_pool[page, :, t % page_size, :] = v_new[i]
        written += 1
    return written
