"""GPU parity with caches past 4 GiB: every block a query reads sits beyond byte
2^32 of its cache (bf16: 60,000 blocks of 73,728 B; FP8: 120,000 blocks of
36,864 B of codes), so a cache offset truncated to 32 bits anywhere in the
decode, sparse, append or FP8 kernels would read or write the wrong rows. The
oracle sees the same rows through a compact cache and the block table mapped
back to it, which is the same attention."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
import workloads as wl
from oracle import append as oracle_append
from oracle import fp8
from tests import cases
from tests.gpu_util import assert_parity

pytestmark = pytest.mark.gpu

BIG_BF16 = 60000       # 60,000 x 73,728 B = 4.42e9 B > 2^32
BIG_FP8 = 120000       # 120,000 x 36,864 B = 4.42e9 B > 2^32


def _say(msg):
    print("[case] " + msg, flush=True)


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def high_ids(n_compact, n_big, seed):
    """Device block id of each compact block: the top of the big cache, shuffled."""
    rng = np.random.default_rng(seed)
    return (n_big - 1 - rng.permutation(n_compact)).astype(np.int64)


def big_table(table, ids):
    return np.where(table >= 0, ids[np.maximum(table, 0)], -1).astype(np.int32)


@pytest.fixture(scope="module")
def big_bf16():
    assert torch.cuda.is_available()
    kc = torch.empty((BIG_BF16, wl.PAGE, wl.D_QK), dtype=torch.bfloat16, device="cuda")
    yield kc
    del kc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lens,s_q,h_q", [([300, 1000, 5], 1, 16), ([700, 64, 1500], 2, 32)])
def test_large_cache_decode_bf16(big_bf16, lens, s_q, h_q):
    _say("large bf16 decode lens=%s s_q=%d h_q=%d" % (lens, s_q, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=31 + h_q, poison=False)
    ids = high_ids(inp.kcache.shape[0], BIG_BF16, 5)
    kc = big_bf16
    kc[torch.from_numpy(ids).cuda()] = bf16_dev(inp.kcache)
    table = torch.from_numpy(big_table(inp.block_table, ids)).cuda()
    lens_d = torch.from_numpy(inp.cache_seqlens).cuda()
    meta, splits = mla.mla_get_metadata(lens_d, h_q, s_q)
    out, lse = mla.mla_decode_fwd(bf16_dev(inp.q), kc, table, lens_d, inp.softmax_scale, meta, splits,
                                  causal=inp.causal)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_inputs(inp)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "large bf16 %s" % (lens,))


def test_large_cache_sparse(big_bf16):
    _say("large sparse")
    rng = np.random.default_rng(9)
    inp = cases.small_batch([900, 3000], s_q=1, h_q=16, seed=41, causal=False, poison=False)
    topk = 256
    idx = np.stack([rng.choice(int(L), size=topk, replace=False) for L in inp.cache_seqlens])[:, None, :]
    idx = idx.astype(np.int32)
    counts = np.full((2,), topk, dtype=np.int32)
    ids = high_ids(inp.kcache.shape[0], BIG_BF16, 6)
    kc = big_bf16
    kc[torch.from_numpy(ids).cuda()] = bf16_dev(inp.kcache)
    table = torch.from_numpy(big_table(inp.block_table, ids)).cuda()
    cnt = torch.from_numpy(counts).cuda()
    meta, splits = mla.mla_get_metadata_sparse(cnt, 2, 1, 16, topk)
    out, lse = mla.mla_decode_sparse_fwd(bf16_dev(inp.q), kc, table, torch.from_numpy(idx).cuda(), cnt,
                                         inp.softmax_scale, meta, splits)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode_sparse(inp.q, inp.kcache, inp.block_table, idx, counts, inp.softmax_scale)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "large sparse")


def test_large_cache_append_bf16(big_bf16):
    _say("large bf16 append")
    inp = cases.small_batch([200, 1000, 70], s_q=1, h_q=16, seed=51, poison=False)
    rng = np.random.default_rng(3)
    new = wl.f32_to_bf16_bits(rng.standard_normal((3, 100, wl.D_QK)).astype(np.float32))
    ids = high_ids(inp.kcache.shape[0], BIG_BF16, 7)
    kc = big_bf16
    ids_d = torch.from_numpy(ids).cuda()
    kc[ids_d] = bf16_dev(inp.kcache)
    table = torch.from_numpy(big_table(inp.block_table, ids)).cuda()
    mla.mla_append_kv(kc, table, torch.from_numpy(inp.cache_seqlens).cuda(), bf16_dev(new))
    torch.cuda.synchronize()
    got = kc[ids_d].view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle_append.append_rows(inp.kcache, inp.block_table, inp.cache_seqlens, new)
    assert np.array_equal(got, want)


@pytest.fixture(scope="module")
def big_fp8():
    assert torch.cuda.is_available()
    codes = torch.empty((BIG_FP8, wl.PAGE, wl.D_QK), dtype=torch.uint8, device="cuda")
    scales = torch.empty((BIG_FP8, wl.PAGE), dtype=torch.float32, device="cuda")
    yield codes, scales
    del codes, scales
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lens,s_q,h_q", [([300, 1000, 5], 1, 16), ([700, 64, 1500], 1, 64)])
def test_large_cache_decode_fp8(big_fp8, lens, s_q, h_q):
    _say("large fp8 decode lens=%s s_q=%d h_q=%d" % (lens, s_q, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=61 + h_q, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    ids = high_ids(inp.kcache.shape[0], BIG_FP8, 8)
    ids_d = torch.from_numpy(ids).cuda()
    dc, ds = big_fp8
    dc[ids_d] = torch.from_numpy(codes).cuda()
    ds[ids_d] = torch.from_numpy(scales).cuda()
    table = torch.from_numpy(big_table(inp.block_table, ids)).cuda()
    lens_d = torch.from_numpy(inp.cache_seqlens).cuda()
    meta, splits = mla.mla_get_metadata_fp8(lens_d, h_q, s_q)
    out, lse = mla.mla_decode_fp8_fwd(bf16_dev(inp.q), dc, ds, table, lens_d, inp.softmax_scale, meta, splits,
                                      causal=inp.causal)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode_fp8(inp.q, codes, scales, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                                   inp.causal)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "large fp8 %s" % (lens,))


def test_large_cache_append_fp8(big_fp8):
    _say("large fp8 append")
    inp = cases.small_batch([200, 1000, 70], s_q=1, h_q=16, seed=71, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    rng = np.random.default_rng(4)
    new = wl.f32_to_bf16_bits(rng.standard_normal((3, 100, wl.D_QK)).astype(np.float32))
    ids = high_ids(inp.kcache.shape[0], BIG_FP8, 9)
    ids_d = torch.from_numpy(ids).cuda()
    dc, ds = big_fp8
    dc[ids_d] = torch.from_numpy(codes).cuda()
    ds[ids_d] = torch.from_numpy(scales).cuda()
    table = torch.from_numpy(big_table(inp.block_table, ids)).cuda()
    mla.mla_append_kv_fp8(dc, ds, table, torch.from_numpy(inp.cache_seqlens).cuda(), bf16_dev(new))
    torch.cuda.synchronize()
    rc, rs = fp8.append_rows_fp8(codes, scales, inp.block_table, inp.cache_seqlens, new)
    assert np.array_equal(dc[ids_d].cpu().numpy(), rc)
    assert np.array_equal(ds[ids_d].cpu().numpy().view(np.uint32), rs.view(np.uint32))
