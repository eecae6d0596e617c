"""Pins of the append oracle and property tests of the block pool (CPU only).

The append oracle (oracle/append.py) writes new rows into the paged cache. It
is pinned here by facts that do not depend on it: the rows read back through a
separately written gather are the new rows; nothing else in the cache moves;
appending the last s_new rows of a seeded cache into a cache where they were
wiped restores it byte for byte, and the decode oracle then gives bitwise the
same result; planted mistakes in a copy of the oracle fail these checks.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads as wl
from oracle import append as app
from oracle import mla_decode


def gather_sequence(kcache, table_row, length, page=64):
    """Rows 0..length-1 of one sequence, read block by block (an independent path)."""
    nb = (length + page - 1) // page
    if nb == 0:
        return kcache[:0].reshape(0, kcache.shape[2])
    rows = np.concatenate([kcache[int(table_row[j])] for j in range(nb)], axis=0)
    return rows[:length]


def make_case(lens, s_new, seed, width=576, spare=3):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    nb = (lens + 63) // 64
    nblocks = int(nb.sum()) + spare
    perm = rng.permutation(nblocks).astype(np.int32)
    table = np.full((len(lens), max(1, int(nb.max()))), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[off:off + n]
        off += n
    kcache = rng.integers(0, 2 ** 16, size=(nblocks, 64, width), dtype=np.uint16)
    new_rows = rng.integers(0, 2 ** 16, size=(len(lens), s_new, width), dtype=np.uint16)
    return kcache, table, lens, new_rows


CASES = [([64, 200, 1], 1), ([130, 64, 5], 2), ([300, 70], 64), ([129, 1, 3000], 100), ([10], 16)]


@pytest.mark.parametrize("lens,s_new", CASES)
def test_rows_land_at_the_last_positions(lens, s_new):
    kcache, table, L, new = make_case(lens, s_new, seed=sum(lens) + s_new)
    got = app.append_rows(kcache, table, L, new)
    for b, n in enumerate(L):
        seq = gather_sequence(got, table[b], int(n))
        k = min(s_new, int(n))                       # rows that fit (the first s_new - k have position < 0)
        assert np.array_equal(seq[int(n) - k:], new[b, s_new - k:]), "new rows not at the tail of sequence %d" % b
        before = gather_sequence(kcache, table[b], int(n))
        assert np.array_equal(seq[:int(n) - k], before[:int(n) - k]), "older rows of sequence %d changed" % b


@pytest.mark.parametrize("lens,s_new", CASES)
def test_nothing_else_changes(lens, s_new):
    kcache, table, L, new = make_case(lens, s_new, seed=7 * sum(lens) + s_new)
    got = app.append_rows(kcache, table, L, new)
    written = np.zeros(kcache.shape[:2], dtype=bool)
    for b, n in enumerate(L):
        for t in range(max(0, int(n) - s_new), int(n)):
            written[table[b, t // 64], t % 64] = True
    assert np.array_equal(got[~written], kcache[~written])
    assert written.sum() == sum(min(s_new, int(n)) for n in L)


def test_append_restores_a_cache_and_its_decode():
    """Wipe the last s_q rows of every sequence of a seeded workload (NaN), append
    them back: the cache is restored byte for byte and the decode is unchanged."""
    inp = wl.make_workload("tiny", poison=True)
    s_new = 3
    new = np.stack([gather_sequence(inp.kcache, inp.block_table[b], int(n))[int(n) - s_new:]
                    for b, n in enumerate(inp.cache_seqlens)])
    wiped = inp.kcache.copy()
    for b, n in enumerate(inp.cache_seqlens):
        for t in range(int(n) - s_new, int(n)):
            wiped[inp.block_table[b, t // 64], t % 64] = wl.BF16_NAN
    restored = app.append_rows(wiped, inp.block_table, inp.cache_seqlens, new)
    assert np.array_equal(restored, inp.kcache)
    o1, l1 = mla_decode(inp.q, inp.kcache, inp.block_table, inp.cache_seqlens, inp.softmax_scale, inp.causal)
    o2, l2 = mla_decode(inp.q, restored, inp.block_table, inp.cache_seqlens, inp.softmax_scale, inp.causal)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _planted(kind):
    """A copy of the oracle with one plausible mistake."""
    def f(kcache, block_table, cache_seqlens, new_rows, page=64):
        out = np.array(kcache, copy=True)
        B, s_new = new_rows.shape[0], new_rows.shape[1]
        for b in range(B):
            length = int(cache_seqlens[b])
            for i in range(s_new):
                pos = length - s_new + i
                if kind == "off_by_one":
                    pos += 1
                if pos < 0 and kind != "no_skip":
                    continue
                blk, row = pos // page, pos % page
                if kind == "row_from_block_index":
                    row = blk % page
                if kind == "table_not_used":
                    blk_id = blk
                else:
                    blk_id = int(block_table[b, blk])
                if kind == "first_512_only":
                    out[blk_id, row, :512] = new_rows[b, i, :512]
                elif kind == "reversed_rows":
                    out[blk_id, row, :] = new_rows[b, s_new - 1 - i, :]
                else:
                    out[blk_id, row, :] = new_rows[b, i, :]
        return out
    return f


@pytest.mark.parametrize("kind", ["off_by_one", "no_skip", "row_from_block_index", "table_not_used",
                                  "first_512_only", "reversed_rows"])
def test_planted_mistakes_are_caught(kind):
    bad = _planted(kind)
    caught = False
    for lens, s_new in CASES:
        kcache, table, L, new = make_case(lens, s_new, seed=sum(lens) + s_new)
        try:
            got = bad(kcache, table, L, new)
        except (IndexError, ValueError):
            caught = True
            break
        if not np.array_equal(got, app.append_rows(kcache, table, L, new)):
            # the pins above must see the difference, not just the reference comparison
            for b, n in enumerate(L):
                seq = gather_sequence(got, table[b], int(n))
                k = min(s_new, int(n))
                if not np.array_equal(seq[int(n) - k:], new[b, s_new - k:]):
                    caught = True
            written = np.zeros(kcache.shape[:2], dtype=bool)
            for b, n in enumerate(L):
                for t in range(max(0, int(n) - s_new), int(n)):
                    written[table[b, t // 64], t % 64] = True
            if not np.array_equal(got[~written], kcache[~written]):
                caught = True
        if caught:
            break
    assert caught, kind
