"""Plain CPU oracle for the cache append (test infrastructure).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this module. It shares nothing with the HIP library.

What it computes: at each decode step the new tokens' entries are added to the
cache ("OpenSourceWeek Day 1: FlashMLA", bibleofai.com, "How KV Caching
Works?"); the cache is paged, a sequence's token t living in row t % 64 of
its block block_table[b][t // 64] (same page, "Key Highlights", block size 64;
FlashMLA explainer, theflyingbirds.in, section 4.3.2 "Paged KV Cache").
Reading where the pages are silent (the same one the decode oracle takes): the
s_new new tokens of sequence b are its last s_new positions, so new row i goes
to position cache_seqlens[b] - s_new + i, and a position below 0 (a sequence
shorter than s_new) is not written.
"""
from __future__ import annotations

import numpy as np


def append_rows(kcache, block_table, cache_seqlens, new_rows, page: int = 64):
    """Return a copy of kcache (any dtype, [nblocks, page, width]) with
    new_rows [B, s_new, width] written at their positions; nothing else changes."""
    out = np.array(kcache, copy=True)
    B, s_new = new_rows.shape[0], new_rows.shape[1]
    for b in range(B):
        length = int(cache_seqlens[b])
        for i in range(s_new):
            pos = length - s_new + i
            if pos < 0:
                continue
            out[int(block_table[b, pos // page]), pos % page, :] = new_rows[b, i, :]
    return out
