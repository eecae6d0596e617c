"""GPU parity of the sparse (top-k index) decode against the sparse CPU oracle,
through the C ABI: random lists with padding and short counts, NaN in every
cache row no list names, several head counts and new-token counts, extreme
plans, empty lists, and the benchmark workload at full size on sampled rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
import workloads as wl
from tests.gpu_util import assert_parity, rel_rms

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def make(lens, s_q, h_q, topk, seed, pad_frac=0.1, short=True):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    dec = wl.build_inputs(lens, s_q, h_q, rng, name="sparse", causal=False, poison=True)
    B = len(lens)
    idx = np.full((B, s_q, topk), -1, dtype=np.int32)
    counts = np.zeros((B * s_q,), dtype=np.int32)
    for b in range(B):
        for i in range(s_q):
            n = min(topk, int(lens[b]))
            pick = rng.choice(int(lens[b]), size=n, replace=False) if n else np.zeros(0, np.int32)
            pad = rng.random(n) < pad_frac
            pick = np.where(pad, -1, pick)
            k = int(rng.integers(max(0, n - 5), n + 1)) if (short and n) else n
            idx[b, i, :k] = pick[:k]
            counts[b * s_q + i] = k
    return dec, idx, counts


def run(dec, idx, counts, num_units=None):
    B, s_q, h_q = dec.batch, dec.s_q, dec.h_q
    topk = idx.shape[2]
    lens = torch.from_numpy(counts).cuda()
    meta, splits = mla.mla_get_metadata_sparse(lens, B, s_q, h_q, topk, num_units=num_units)
    out, lse = mla.mla_decode_sparse_fwd(bf16_dev(dec.q), bf16_dev(dec.kcache), torch.from_numpy(dec.block_table).cuda(),
                                         torch.from_numpy(idx).cuda(), lens, dec.softmax_scale, meta, splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def ref(dec, idx, counts):
    return oracle.mla_decode_sparse(dec.q, dec.kcache, dec.block_table, idx, counts, dec.softmax_scale)


CASES = [([64, 200], 1, 16, 32), ([300, 70, 1000], 2, 16, 100), ([2000], 1, 32, 2048), ([500, 64], 3, 16, 7),
         ([129, 40, 3, 900], 1, 128, 64), ([5000, 300], 1, 16, 1)]


@pytest.mark.parametrize("lens,s_q,h_q,topk", CASES)
def test_sparse_parity(lens, s_q, h_q, topk):
    _say("sparse lens=%s s_q=%d h_q=%d topk=%d" % (lens, s_q, h_q, topk))
    dec, idx, counts = make(lens, s_q, h_q, topk, seed=sum(lens) + topk)
    out, lse = run(dec, idx, counts)
    ro, rl = ref(dec, idx, counts)
    assert_parity(out, lse, ro, rl, "sparse %s" % (lens,))
    print("rel rms %.2e" % rel_rms(out, ro))


def test_sparse_empty_and_all_padding():
    _say("sparse empty lists")
    dec, idx, counts = make([300, 100, 50], 1, 16, 40, seed=3)
    idx[1] = -1                          # all padding
    counts[2] = 0                        # nothing in use
    out, lse = run(dec, idx, counts)
    ro, rl = ref(dec, idx, counts)
    assert_parity(out, lse, ro, rl, "empty")
    assert (out[1:] == 0).all() and np.isneginf(lse[1:]).all()


@pytest.mark.parametrize("units", [4, 7, 40, 600])
def test_sparse_plan_extremes(units):
    _say("sparse units=%d" % units)
    dec, idx, counts = make([900, 64, 2000], 1, 16, 1024, seed=units)
    out, lse = run(dec, idx, counts, num_units=units)
    ro, rl = ref(dec, idx, counts)
    assert_parity(out, lse, ro, rl, "units %d" % units)


def test_sparse_full_list_matches_dense_decode():
    """A list naming every cached position in order gives the dense decode's answer."""
    _say("sparse full list vs dense")
    inp = wl.make_workload("tiny", poison=True)
    inp.causal = False
    topk = int(inp.cache_seqlens.max())
    idx = np.full((inp.batch, 1, topk), -1, dtype=np.int32)
    for b in range(inp.batch):
        idx[b, 0, :inp.cache_seqlens[b]] = np.arange(inp.cache_seqlens[b])
    counts = inp.cache_seqlens.copy()
    out, lse = run(inp, idx, counts)
    ro, rl = oracle.mla_decode(inp.q, inp.kcache, inp.block_table, inp.cache_seqlens, inp.softmax_scale, False)
    assert_parity(out, lse, ro, rl, "full list")


def test_sparse_bench_workload_sampled_rows():
    """The benchmark's sparse workload at full size; the oracle checks a sample of rows."""
    _say("sparse bench workload")
    sp = wl.make_sparse(poison=True)
    dec = sp.dec
    out, lse = run(dec, sp.indices, sp.counts)
    rng = np.random.default_rng(0)
    for b in rng.choice(dec.batch, size=4, replace=False):
        sub = wl.subset(dec, [b])
        ro, rl = oracle.mla_decode_sparse(sub.q, sub.kcache, sub.block_table, sp.indices[[b]], sp.counts[[b]],
                                          dec.softmax_scale)
        assert_parity(out[[b]], lse[[b]], ro, rl, "bench row %d" % b)
