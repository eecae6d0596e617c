"""The two-stage form of every decode call: the decode kernel alone (the *_splits
entry points) followed by mla_combine_splits on the same plan and workspace gives
bit for bit what the one-call form gives -- bf16 cache (16- and 64-row
workgroups), FP8 cache (both kernels) and sparse lists -- for plans where every
sequence is split and plans where most are not. One case per cache type is also
checked against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
from oracle import fp8
from tests import cases
from tests.gpu_util import assert_parity, to_device
from tests.test_gpu_sparse import make as make_sparse

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    mla.load_library()


def _say(msg):
    print("\n[case] " + msg, flush=True)


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), what


SHAPES = [([5000, 64, 900, 3000, 1], 1, 16), ([2100, 700, 64, 4000], 2, 64), ([3000, 129], 1, 128)]


@pytest.mark.parametrize("lens,s_q,h_q", SHAPES)
@pytest.mark.parametrize("few_units", [False, True])
def test_bf16_splits_then_combine_is_the_one_call(lens, s_q, h_q, few_units):
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=300 + h_q)
    dev = to_device(inp)
    units = len(lens) + 1 if few_units else None
    meta, splits = mla.mla_get_metadata(dev["cache_seqlens"], h_q, s_q, num_units=units)
    _say("bf16 lens=%s s_q=%d h_q=%d units=%s" % (lens, s_q, h_q, units))
    o1, l1 = mla.mla_decode_fwd(dev["q"], dev["kcache"], dev["block_table"], dev["cache_seqlens"], inp.softmax_scale,
                                meta, splits, causal=True)
    o2, l2, ws = mla.mla_decode_fwd_splits(dev["q"], dev["kcache"], dev["block_table"], dev["cache_seqlens"],
                                           inp.softmax_scale, meta, splits, causal=True)
    mla.mla_combine_splits(splits, s_q, h_q, int(meta.shape[0]), o2, l2, ws)
    torch.cuda.synchronize()
    _same(o1, o2, "out")
    _same(l1, l2, "lse")
    if not few_units and h_q == 16:
        ref_out, ref_lse = oracle.decode_inputs(inp)
        assert_parity(o2.float().cpu().numpy(), l2.cpu().numpy(), ref_out, ref_lse, "two-stage bf16")


@pytest.mark.parametrize("lens,s_q,h_q", SHAPES)
@pytest.mark.parametrize("few_units", [False, True])
def test_fp8_splits_then_combine_is_the_one_call(lens, s_q, h_q, few_units):
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=400 + h_q, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    dev = to_device(inp)
    c, sc = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    units = len(lens) + 1 if few_units else None
    meta, splits = mla.mla_get_metadata_fp8(dev["cache_seqlens"], h_q, s_q, num_units=units)
    _say("fp8 lens=%s s_q=%d h_q=%d units=%s" % (lens, s_q, h_q, units))
    o1, l1 = mla.mla_decode_fp8_fwd(dev["q"], c, sc, dev["block_table"], dev["cache_seqlens"], inp.softmax_scale,
                                    meta, splits, causal=True)
    o2, l2, ws = mla.mla_decode_fp8_fwd_splits(dev["q"], c, sc, dev["block_table"], dev["cache_seqlens"],
                                               inp.softmax_scale, meta, splits, causal=True)
    mla.mla_combine_splits(splits, s_q, h_q, int(meta.shape[0]), o2, l2, ws)
    torch.cuda.synchronize()
    _same(o1, o2, "out")
    _same(l1, l2, "lse")
    if not few_units and h_q == 64:
        ref_out, ref_lse = oracle.mla_decode_fp8(inp.q, codes, scales, inp.block_table, inp.cache_seqlens,
                                                 inp.softmax_scale, True)
        assert_parity(o2.float().cpu().numpy(), l2.cpu().numpy(), ref_out, ref_lse, "two-stage fp8")


@pytest.mark.parametrize("lens,s_q,h_q,topk", [([3000, 70, 1000], 2, 16, 1000), ([2000, 600], 1, 64, 2048)])
@pytest.mark.parametrize("few_units", [False, True])
def test_sparse_splits_then_combine_is_the_one_call(lens, s_q, h_q, topk, few_units):
    d, idx, counts = make_sparse(lens, s_q, h_q, topk, seed=500 + topk)
    B = d.batch
    dev = to_device(d)
    lens_d = torch.from_numpy(counts).cuda()
    idx_d = torch.from_numpy(idx).cuda()
    units = B * s_q + 1 if few_units else None
    meta, splits = mla.mla_get_metadata_sparse(lens_d, B, s_q, h_q, topk, num_units=units)
    _say("sparse lens=%s s_q=%d h_q=%d topk=%d units=%s" % (lens, s_q, h_q, topk, units))
    o1, l1 = mla.mla_decode_sparse_fwd(dev["q"], dev["kcache"], dev["block_table"], idx_d, lens_d, d.softmax_scale,
                                       meta, splits)
    o2, l2, ws = mla.mla_decode_sparse_fwd_splits(dev["q"], dev["kcache"], dev["block_table"], idx_d, lens_d,
                                                  d.softmax_scale, meta, splits)
    mla.mla_combine_splits(splits, 1, h_q, int(meta.shape[0]), o2, l2, ws)
    torch.cuda.synchronize()
    _same(o1, o2, "out")
    _same(l1, l2, "lse")
    if not few_units and h_q == 16:
        ref_out, ref_lse = oracle.mla_decode_sparse(d.q, d.kcache, d.block_table, idx, counts, d.softmax_scale)
        assert_parity(o2.float().cpu().numpy(), l2.cpu().numpy(), ref_out, ref_lse, "two-stage sparse")
