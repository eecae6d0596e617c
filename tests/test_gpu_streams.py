"""The decode calls keep no state between calls: two batches decoded at the same time
on two streams (default priority), each with its own plan and workspace, give bit for
bit what each gives alone -- for the 16-row and the 64-row bf16 kernels and the FP8
cache -- and the first batch also matches the oracle."""
from __future__ import annotations

import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
from oracle import fp8
from tests import cases
from tests.gpu_util import assert_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    mla.load_library()


def _say(msg):
    print("\n[case] " + msg, flush=True)


def _batches(h_q, s_q):
    a = cases.small_batch([3000, 700, 64, 1500], s_q=s_q, h_q=h_q, seed=610 + h_q, poison=False)
    b = cases.small_batch([129, 4000, 900], s_q=s_q, h_q=h_q, seed=620 + h_q, poison=False)
    return a, b


def _decoder(inp, use_fp8):
    """A closure that plans and decodes inp on the current stream into fresh tensors."""
    dev = to_device(inp)
    if use_fp8:
        codes, scales = fp8.quantize_rows(inp.kcache)
        c, sc = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()

    def run():
        if use_fp8:
            meta, splits = mla.mla_get_metadata_fp8(dev["cache_seqlens"], inp.h_q, inp.s_q)
            return mla.mla_decode_fp8_fwd(dev["q"], c, sc, dev["block_table"], dev["cache_seqlens"],
                                          inp.softmax_scale, meta, splits, causal=True)
        meta, splits = mla.mla_get_metadata(dev["cache_seqlens"], inp.h_q, inp.s_q)
        return mla.mla_decode_fwd(dev["q"], dev["kcache"], dev["block_table"], dev["cache_seqlens"],
                                  inp.softmax_scale, meta, splits, causal=True)
    return run


@pytest.mark.parametrize("h_q,s_q,use_fp8", [(16, 1, False), (128, 1, False), (64, 2, False), (16, 1, True),
                                            (128, 1, True)])
def test_two_streams_at_once_match_each_alone(h_q, s_q, use_fp8):
    a, b = _batches(h_q, s_q)
    run_a, run_b = _decoder(a, use_fp8), _decoder(b, use_fp8)
    _say("two streams h_q=%d s_q=%d fp8=%d: each alone" % (h_q, s_q, use_fp8))
    oa, la = run_a()
    ob, lb = run_b()
    torch.cuda.synchronize()
    _say("both at once")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(sa):
            ra = run_a()
        with torch.cuda.stream(sb):
            rb = run_b()
        torch.cuda.synchronize()
        assert torch.equal(ra[0].view(torch.int16), oa.view(torch.int16)) and torch.equal(ra[1], la)
        assert torch.equal(rb[0].view(torch.int16), ob.view(torch.int16)) and torch.equal(rb[1], lb)
    if use_fp8:
        codes, scales = fp8.quantize_rows(a.kcache)
        ref_out, ref_lse = oracle.mla_decode_fp8(a.q, codes, scales, a.block_table, a.cache_seqlens,
                                                 a.softmax_scale, True)
    else:
        ref_out, ref_lse = oracle.decode_inputs(a)
    assert_parity(oa.float().cpu().numpy(), la.cpu().numpy(), ref_out, ref_lse, "stream A")
