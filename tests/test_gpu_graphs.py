"""HIP-graph capture of the FP8, sparse and append paths, as the benchmark runs them: every
replay gives exactly the eager result, with eager work and synchronisations between the
replays, and the result matches the oracle."""
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


def _say(msg):
    print("[case] " + msg, flush=True)


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def replay_check(run, outputs, reset):
    """Run eagerly, capture, then replay three times (reset() -- eager fill or copy kernels --
    before each replay) and compare each replay and the eager run after it bitwise."""
    reset()
    run()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        run()
    for rep in range(3):
        reset()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, refs):
            assert torch.equal(t, r), "replay %d differs" % rep
        reset()
        run()
        torch.cuda.synchronize()
        for t, r in zip(outputs, refs):
            assert torch.equal(t, r), "eager run after replay %d differs" % rep


@pytest.mark.parametrize("lens,s_q,h_q", [([500, 70, 1300], 1, 16), ([300, 2000, 64], 1, 128)])
def test_fp8_graph_replays(lens, s_q, h_q):
    _say("fp8 graph lens=%s h_q=%d" % (lens, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=sum(lens) + 5, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    B = len(lens)
    q, dc, ds = bf16_dev(inp.q), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    table, lens_d = torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.cache_seqlens).cuda()
    sizes = mla.mla_fp8_plan_sizes(B, s_q, h_q)
    units = sizes["num_units"]
    meta = torch.empty((units, mla.META_INTS), dtype=torch.int32, device="cuda")
    splits = torch.empty((B + 1,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s_q, h_q, mla.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device="cuda")
    ws = torch.empty((sizes["workspace_bytes"],), dtype=torch.uint8, device="cuda")

    def run():
        mla.mla_get_metadata_fp8(lens_d, h_q, s_q, num_units=units, tile_meta=meta, num_splits=splits)
        mla.mla_decode_fp8_fwd(q, dc, ds, table, lens_d, inp.softmax_scale, meta, splits, causal=True, out=out,
                               lse=lse, workspace=ws)

    replay_check(run, [out, lse], lambda: [t.zero_() for t in (out, lse, meta, ws)])
    ro, rl = oracle.mla_decode_fp8(inp.q, codes, scales, inp.block_table, inp.cache_seqlens, inp.softmax_scale, True)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "fp8 graph")


def test_sparse_graph_replays():
    _say("sparse graph")
    rng = np.random.default_rng(21)
    inp = cases.small_batch([900, 3000, 64], s_q=2, h_q=16, seed=22, causal=False, poison=False)
    topk = 300
    idx = np.full((3, 2, topk), -1, dtype=np.int32)
    counts = np.zeros((6,), dtype=np.int32)
    for b in range(3):
        for i in range(2):
            n = min(topk, int(inp.cache_seqlens[b]))
            idx[b, i, :n] = rng.choice(int(inp.cache_seqlens[b]), size=n, replace=False)
            counts[2 * b + i] = n - (b % 2)
    q, kc, table = bf16_dev(inp.q), bf16_dev(inp.kcache), torch.from_numpy(inp.block_table).cuda()
    idx_d, cnt = torch.from_numpy(idx).cuda(), torch.from_numpy(counts).cuda()
    sizes = mla.mla_sparse_plan_sizes(3, 2, 16, topk)
    units = sizes["num_units"]
    meta = torch.empty((units, mla.META_INTS), dtype=torch.int32, device="cuda")
    splits = torch.empty((7,), dtype=torch.int32, device="cuda")
    out = torch.empty((3, 2, 16, mla.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((3, 2, 16), dtype=torch.float32, device="cuda")
    ws = torch.empty((sizes["workspace_bytes"],), dtype=torch.uint8, device="cuda")

    def run():
        mla.mla_get_metadata_sparse(cnt, 3, 2, 16, topk, num_units=units, tile_meta=meta, num_splits=splits)
        mla.mla_decode_sparse_fwd(q, kc, table, idx_d, cnt, inp.softmax_scale, meta, splits, out=out, lse=lse,
                                  workspace=ws)

    replay_check(run, [out, lse], lambda: [t.zero_() for t in (out, lse, meta, ws)])
    ro, rl = oracle.mla_decode_sparse(inp.q, inp.kcache, inp.block_table, idx, counts, inp.softmax_scale)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "sparse graph")


def test_append_graph_replays():
    """The bf16 and FP8 appends captured in one graph: each replay rewrites the same rows."""
    _say("append graph")
    inp = cases.small_batch([200, 1000, 70], s_q=1, h_q=16, seed=23, poison=False)
    rng = np.random.default_rng(24)
    new = wl.f32_to_bf16_bits(rng.standard_normal((3, 100, wl.D_QK)).astype(np.float32))
    codes, scales = fp8.quantize_rows(inp.kcache)
    kc, dc, ds = bf16_dev(inp.kcache), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    table, lens_d, rows = torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.cache_seqlens).cuda(), bf16_dev(new)

    def run():
        mla.mla_append_kv(kc, table, lens_d, rows)
        mla.mla_append_kv_fp8(dc, ds, table, lens_d, rows)

    kc0, dc0, ds0 = kc.clone(), dc.clone(), ds.clone()
    replay_check(run, [kc, dc, ds], lambda: [t.copy_(t0) for t, t0 in ((kc, kc0), (dc, dc0), (ds, ds0))])
    assert np.array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle_append.append_rows(inp.kcache, inp.block_table, inp.cache_seqlens, new))
    rc, rs = fp8.append_rows_fp8(codes, scales, inp.block_table, inp.cache_seqlens, new)
    assert np.array_equal(dc.cpu().numpy(), rc)
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), rs.view(np.uint32))
