"""Host tests of the paged block pool and of the append entry point's argument
checks (no GPU). The pool is checked step by step against a plain Python model
of the same rules: blocks handed out lowest id first, freed blocks reused last
freed first, a slot's kept blocks never move, a failed reservation changes
nothing."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import mla_paged_latent_amd as mla

PAGE = 64


class Model:
    def __init__(self, nblocks, max_seqs, cap):
        self.free = list(range(nblocks - 1, -1, -1))    # the last entry goes out next
        self.own = [[] for _ in range(max_seqs)]
        self.lens = [0] * max_seqs
        self.cap = cap

    def reserve(self, seq, n):
        need = (n + PAGE - 1) // PAGE
        if need > self.cap:
            return "invalid"
        own = self.own[seq]
        if need > len(own):
            if len(self.free) < need - len(own):
                return "out_of_blocks"
            while len(own) < need:
                own.append(self.free.pop())
        else:
            while len(own) > need:
                self.free.append(own.pop())
        self.lens[seq] = n
        return "ok"


@pytest.fixture(scope="module")
def built():
    if not mla.LIB_PATH.exists():
        from mla_paged_latent_amd import build
        build.build()
    return mla.load_library()


def check_against(pool, model, max_seqs, cap):
    table, lens = pool.table(np.arange(max_seqs), cap)
    for s in range(max_seqs):
        want = model.own[s] + [-1] * (cap - len(model.own[s]))
        assert table[s].tolist() == want, s
        assert lens[s] == model.lens[s]
    assert pool.free_blocks() == len(model.free)
    used = table[table >= 0]
    assert len(np.unique(used)) == used.size, "a block belongs to two slots"
    assert used.size + pool.free_blocks() == pool.nblocks


def test_fresh_pool_hands_out_lowest_ids_first(built):
    p = mla.BlockPool(10, 3, 6)
    p.reserve(1, 130)
    p.reserve(0, 1)
    t, lens = p.table([0, 1, 2], 6)
    assert t[1, :3].tolist() == [0, 1, 2] and t[0, 0] == 3 and (t[2] == -1).all()
    assert lens.tolist() == [1, 130, 0]


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_follow_the_model(built, seed):
    rng = np.random.default_rng(seed)
    nblocks, max_seqs, cap = 40, 6, 12
    p = mla.BlockPool(nblocks, max_seqs, cap)
    m = Model(nblocks, max_seqs, cap)
    for _ in range(300):
        seq = int(rng.integers(0, max_seqs))
        op = rng.random()
        if op < 0.15:
            n = 0
        elif op < 0.3:
            n = max(0, m.lens[seq] - int(rng.integers(0, 200)))
        else:
            n = m.lens[seq] + int(rng.integers(0, 300))
        before = p.table(np.arange(max_seqs), cap)
        want = m.reserve(seq, n)
        if want == "ok":
            p.reserve(seq, n)
        else:
            with pytest.raises(mla.MLAError) as e:
                p.reserve(seq, n)
            assert e.value.status == (-5 if want == "out_of_blocks" else -1)
            after = p.table(np.arange(max_seqs), cap)
            assert all(np.array_equal(x, y) for x, y in zip(before, after)), "failed reserve changed the pool"
        check_against(p, m, max_seqs, cap)


def test_kept_blocks_keep_their_ids(built):
    p = mla.BlockPool(20, 2, 10)
    p.reserve(0, 300)
    first, _ = p.table([0], 10)
    p.reserve(0, 100)                  # shrink to 2 blocks
    p.reserve(1, 64 * 3)               # takes the freed ones (last freed first)
    p.reserve(0, 500)
    after, _ = p.table([0, 1], 10)
    assert after[0, :2].tolist() == first[0, :2].tolist()
    assert after[1, :3].tolist() == [first[0, 2], first[0, 3], first[0, 4]]


def test_table_and_argument_errors(built):
    p = mla.BlockPool(8, 2, 4)
    p.reserve(0, 200)
    with pytest.raises(mla.MLAError):
        p.table([0], 3)                # holds 4 blocks
    with pytest.raises(mla.MLAError):
        p.reserve(2, 10)               # no such slot
    with pytest.raises(mla.MLAError):
        p.reserve(0, -1)
    with pytest.raises(mla.MLAError):
        p.reserve(1, 64 * 4 + 1)       # over max_blocks_per_seq
    p.release(0)
    assert p.free_blocks() == 8
    lib = mla.load_library()
    h = ctypes.c_void_p(None)
    assert lib.mla_block_pool_create(0, 1, 1, ctypes.byref(h)) == -1 and not h.value
    assert lib.mla_block_pool_free_blocks(None) == -1
    assert lib.mla_block_pool_reserve(None, 0, 1) == -1


def test_append_rejects_bad_arguments_before_any_launch(built):
    lib = mla.load_library()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    ok = dict(kcache=fake, nblocks=4, table=fake, max_blocks=2, lens=fake, rows=fake, batch=2, s_new=1)
    for over in [dict(kcache=None), dict(table=None), dict(lens=None), dict(rows=None), dict(nblocks=0),
                 dict(max_blocks=0), dict(batch=0), dict(s_new=0), dict(kcache=odd), dict(rows=odd)]:
        a = dict(ok, **over)
        rc = lib.mla_append_kv(a["kcache"], a["nblocks"], a["table"], a["max_blocks"], a["lens"], a["rows"],
                               a["batch"], a["s_new"], None)
        assert rc == -1, over
