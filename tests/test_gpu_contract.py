"""Decode and append with inputs that break the block-table contract.

The contract (0 <= L_b <= 64 * max_blocks, every used block-table entry in
[0, nblocks)) is the caller's. When it is broken the kernels still read and
write only inside the cache and the table: a decode reads block 0 for an
out-of-range entry or an index past the table (the affected sequence's result
is unspecified), and an append skips such rows. The other sequences of the
batch keep their exact results, and with MLA_DEBUG_CHECK set the decode calls
refuse the batch before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
import workloads as wl
from oracle import append as oracle_append
from tests import cases
from tests.gpu_util import assert_parity, run_library, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    mla.load_library()


def _say(msg):
    print("\n[case] " + msg, flush=True)


def _broken(inp):
    """Sequence 1: an entry of -1 in its used blocks; sequence 2: an entry past the cache;
    sequence 3: a length past what its table row can hold (same table, L = 64 max_blocks + 40)."""
    nb = inp.kcache.shape[0]
    lens = inp.cache_seqlens.copy()
    table = inp.block_table.copy()
    used = (lens + 63) // 64
    table[1, used[1] // 2] = -1
    table[2, used[2] - 1] = nb + 7
    lens[3] = 64 * table.shape[1] + 40
    return wl.DecodeInputs(name=inp.name + "-broken", q=inp.q, kcache=inp.kcache, block_table=table,
                           cache_seqlens=lens, s_q=inp.s_q, h_q=inp.h_q, softmax_scale=inp.softmax_scale,
                           causal=inp.causal), [0, 4, 5]


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (64, 2)])
def test_broken_sequences_leave_the_others_exact(h_q, s_q):
    base = cases.small_batch([900, 2000, 3100, 700, 1500, 64], s_q=s_q, h_q=h_q, seed=40 + h_q)
    inp, good = _broken(base)
    assert mla.mla_check_inputs_host(inp.cache_seqlens, inp.block_table, inp.kcache.shape[0]) == 1
    _say("broken table h_q=%d s_q=%d (the kernels must stay inside the cache and the table)" % (h_q, s_q))
    out, lse, _ = run_library(inp)
    ref_out, ref_lse = oracle.decode_inputs(wl.subset(inp, good))
    assert_parity(out[good], lse[good], ref_out, ref_lse, "valid sequences beside broken ones")
    # the device is fine afterwards: the unbroken batch decodes exactly
    out, lse, _ = run_library(base)
    ref_out, ref_lse = oracle.decode_inputs(base)
    assert_parity(out, lse, ref_out, ref_lse, "unbroken batch after the broken one")


def test_debug_check_refuses_a_broken_batch_before_any_launch(monkeypatch):
    base = cases.small_batch([900, 2000, 3100, 700, 1500, 64], s_q=1, h_q=16, seed=77)
    inp, _ = _broken(base)
    dev = to_device(inp)
    meta, splits = mla.mla_get_metadata(dev["cache_seqlens"], inp.h_q, inp.s_q)
    out = torch.full((inp.batch, 1, 16, 512), 3.0, dtype=torch.bfloat16, device="cuda:0")
    monkeypatch.setenv("MLA_DEBUG_CHECK", "1")
    _say("MLA_DEBUG_CHECK=1, broken table")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_fwd(dev["q"], dev["kcache"], dev["block_table"], dev["cache_seqlens"], inp.softmax_scale,
                           meta, splits, causal=True, out=out)
    assert e.value.status == -1
    torch.cuda.synchronize()
    assert (out.float() == 3.0).all(), "something was written before the check refused the batch"
    gdev = to_device(base)
    gmeta, gsplits = mla.mla_get_metadata(gdev["cache_seqlens"], base.h_q, base.s_q)
    o, l = mla.mla_decode_fwd(gdev["q"], gdev["kcache"], gdev["block_table"], gdev["cache_seqlens"],
                              base.softmax_scale, gmeta, gsplits, causal=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_inputs(base)
    assert_parity(o.float().cpu().numpy(), l.cpu().numpy(), ref_out, ref_lse, "checked unbroken batch")


def test_append_skips_rows_outside_the_cache():
    """Rows whose block-table entry is outside [0, nblocks), or whose position lies past the table,
    are not written; every other row lands exactly where the append oracle puts it."""
    inp = wl.make_append(batch=6, s_new=100, seed=19)
    nb = inp.kcache.shape[0]
    table = inp.block_table.copy()
    lens = inp.cache_seqlens.copy()
    used = (lens + 63) // 64
    table[1, used[1] - 1] = -1                 # the last block of sequence 1: its newest rows are skipped
    table[2, used[2] - 1] = nb + 3             # the last block of sequence 2 is past the cache
    lens[4] = 64 * table.shape[1] + 10         # sequence 4's new rows lie past its table row
    _say("append with a broken table")
    kc = torch.from_numpy(inp.kcache.view(np.int16)).view(torch.bfloat16).cuda()
    rows = torch.from_numpy(inp.new_rows.view(np.int16)).view(torch.bfloat16).cuda()
    mla.mla_append_kv(kc, torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), rows)
    torch.cuda.synchronize()
    got = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    # expected: the oracle's append of the unbroken sequences, then the broken ones' rows whose block is valid
    ok = [0, 3, 5]
    exp = oracle_append.append_rows(inp.kcache, table[ok], lens[ok], inp.new_rows[ok])
    for b in (1, 2, 4):
        for i in range(100):
            tok = int(lens[b]) - 100 + i
            if tok // 64 >= table.shape[1]:
                continue
            page = int(table[b, tok // 64])
            if 0 <= page < nb:
                exp[page, tok % 64] = inp.new_rows[b, i]
    assert np.array_equal(got, exp)
