"""GPU parity of the cache append (bit-exact against the CPU oracle) and an
end-to-end decode step built on the block pool: reserve blocks, append the
new tokens' rows, plan, decode, all through the C ABI, against the oracles."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import workloads as wl
from oracle import append as app
from oracle import mla_decode
from tests.gpu_util import assert_parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def case(lens, s_new, seed, spare=3):
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
    kcache = rng.integers(0, 2 ** 16, size=(nblocks, 64, 576), dtype=np.uint16)
    new = rng.integers(0, 2 ** 16, size=(len(lens), s_new, 576), dtype=np.uint16)
    return kcache, table, lens, new


@pytest.mark.parametrize("lens,s_new", [([64, 200, 1], 1), ([130, 64, 5], 2), ([300, 70], 64),
                                        ([129, 1, 3000], 100), ([10], 16), (list(range(1, 400, 7)), 9)])
def test_append_bit_exact(lens, s_new):
    _say("append lens=%s s_new=%d" % (lens[:6], s_new))
    kcache, table, L, new = case(lens, s_new, seed=len(lens) * 131 + s_new)
    ref = app.append_rows(kcache, table, L, new)
    kc = bf16_dev(kcache)
    mla.mla_append_kv(kc, torch.from_numpy(table).cuda(), torch.from_numpy(L).cuda(), bf16_dev(new))
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), ref)


def test_decode_step_on_the_pool():
    """Three decode steps of a small batch: the pool grows the sequences, the new
    rows are appended, and decode runs over them; each step matches the oracle."""
    _say("pool decode steps")
    rng = np.random.default_rng(5)
    B, s_q, h_q, max_blocks = 4, 2, 16, 16
    pool = mla.BlockPool(40, B, max_blocks)
    nblocks = 40
    host_cache = np.full((nblocks, 64, 576), wl.BF16_NAN, dtype=np.uint16)   # unwritten rows are NaN
    kc = bf16_dev(host_cache)
    lens = np.array([0, 63, 64, 500], dtype=np.int32)
    for b in range(B):                      # prefill: the first lens[b] rows
        pool.reserve(b, int(lens[b]))
    table, got_lens = pool.table(np.arange(B), max_blocks)
    assert np.array_equal(got_lens, lens)
    pre = max(1, int(lens.max()))
    rows = wl.f32_to_bf16_bits(rng.standard_normal((B, pre, 576)).astype(np.float32))
    mla.mla_append_kv(kc, torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), bf16_dev(rows))
    host_cache = app.append_rows(host_cache, table, lens, rows)
    scale = 1.0 / np.sqrt(192.0)
    for step in range(3):
        lens = lens + s_q
        for b in range(B):
            pool.reserve(b, int(lens[b]))
        table, _ = pool.table(np.arange(B), max_blocks)
        new = wl.f32_to_bf16_bits(rng.standard_normal((B, s_q, 576)).astype(np.float32))
        q = wl.f32_to_bf16_bits(rng.standard_normal((B, s_q, h_q, 576)).astype(np.float32))
        t_dev, l_dev = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
        mla.mla_append_kv(kc, t_dev, l_dev, bf16_dev(new))
        host_cache = app.append_rows(host_cache, table, lens, new)
        meta, splits = mla.mla_get_metadata(l_dev, h_q, s_q)
        out, lse = mla.mla_decode_fwd(bf16_dev(q), kc, t_dev, l_dev, scale, meta, splits, causal=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits(kc), host_cache), "step %d: cache differs from the oracle's" % step
        ref_o, ref_l = mla_decode(q, host_cache, table, lens, scale, True)
        assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "step %d" % step)
