"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: |out - ref| <= 1e-2 + 1e-2 |ref| elementwise (out is bf16, ref is the
oracle's float64) and |lse - ref| <= 1e-3. Integer work (the plan) is compared
bit for bit with the library's host planner. Every workload runs at its full
size in the launch configuration the benchmark times; where the oracle would
take too long the comparison uses a sample of whole sequences.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
import workloads as wl
from tests import cases
from tests.gpu_util import assert_parity, rel_rms, run_library, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    mla.load_library()          # raises when the HIP library is not built: no fallback


def _say(msg):
    print("\n[case] " + msg, flush=True)


def _oracle(inp):
    return oracle.decode_inputs(inp)


# ------------------------------------------------------------- hand-derived cases

def _widen_heads(inp, exp_out, exp_lse, h_q=16):
    """The library takes s_q*h_q in multiples of 16: copy each golden query to 16 heads
    (heads are independent, so every copy has the golden answer)."""
    k = h_q // inp.h_q
    q = np.repeat(inp.q, k, axis=2)
    w = wl.DecodeInputs(name=inp.name, q=q, kcache=inp.kcache, block_table=inp.block_table,
                        cache_seqlens=inp.cache_seqlens, s_q=inp.s_q, h_q=inp.h_q * k,
                        softmax_scale=inp.softmax_scale, causal=inp.causal)
    return w, np.repeat(exp_out, k, axis=2), np.repeat(exp_lse, k, axis=2)


def test_golden_closed_forms():
    for inp, exp_out, exp_lse in cases.golden_cases():
        _say("golden " + inp.name)
        inp, exp_out, exp_lse = _widen_heads(inp, exp_out, exp_lse)
        out, lse, _ = run_library(inp)
        assert_parity(out, lse, exp_out, exp_lse, inp.name)


# ------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["tiny", "memory_bound", "long"])
def test_workload_full(name):
    inp = wl.make_workload(name)
    _say("workload %s full, B=%d" % (name, inp.batch))
    out, lse, _ = run_library(inp)
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, name)
    print("rel rms err %.3g" % rel_rms(out, ref_out), flush=True)


@pytest.mark.parametrize("name,nsample", [("compute_bound", 6), ("mixed", 6)])
def test_workload_sampled(name, nsample):
    inp = wl.make_workload(name)
    _say("workload %s full batch on GPU, %d sequences checked" % (name, nsample))
    out, lse, _ = run_library(inp)
    lens = inp.cache_seqlens
    rng = np.random.default_rng(99)
    pick = {int(np.argmin(lens)), int(np.argmax(lens))}
    while len(pick) < nsample:
        pick.add(int(rng.integers(0, inp.batch)))
    pick = sorted(pick)
    ref_out, ref_lse = _oracle(wl.subset(inp, pick))
    assert_parity(out[pick], lse[pick], ref_out, ref_lse, name)
    print("sampled %s rel rms err %.3g" % (pick, rel_rms(out[pick], ref_out)), flush=True)


# ------------------------------------------------------------- shapes and edge cases

SHAPES = [
    # (seqlens, s_q, h_q)
    ([1, 63, 64, 65, 127, 128, 129, 300], 1, 16),
    ([1, 2, 64, 65, 200], 2, 16),            # 32 rows, causal over 2 new tokens
    ([100, 257, 64], 1, 32),
    ([33, 130, 1000], 1, 64),                # 64 rows: the wide kernel
    ([70, 190], 2, 32),                      # 64 rows, causal
    ([5, 129, 700], 1, 128),                 # two head groups of 64
    ([3, 66, 500], 4, 32),                   # 128 rows, causal over 4 new tokens
    ([31, 32, 33, 95, 96, 97, 161], 1, 128),  # block halves cut at every place
    ([1, 40, 3000, 64], 2, 64),              # 128 rows, causal, one long and three short
    ([2, 65, 300], 2, 128),                  # 256 rows: four head groups
    ([7, 64, 0, 900], 3, 64),                # 192 rows, an empty sequence
    ([10, 140], 3, 16),                      # 48 rows: three head groups of 16
    ([1, 2, 3], 4, 16),                      # queries that see no token (L < s_q)
    ([0, 50, 0, 64], 1, 16),                 # empty sequences
    ([4096 + 17], 1, 16),                    # one long sequence, many splits
]


@pytest.mark.parametrize("lens,s_q,h_q", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_shapes(lens, s_q, h_q):
    _say("shape lens=%s s_q=%d h_q=%d" % (lens, s_q, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=sum(lens) + s_q * h_q)
    out, lse, _ = run_library(inp)
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, str(lens))


def test_non_causal_multi_token():
    inp = cases.small_batch([10, 90, 200], s_q=2, h_q=16, seed=5, causal=False)
    _say("non-causal s_q=2")
    out, lse, _ = run_library(inp)
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, "non-causal")


@pytest.mark.parametrize("h_q,units", [(16, 6), (16, 7), (16, 40), (16, 2000), (64, 3), (64, 300), (128, 1),
                                        (128, 2), (128, 7), (128, 300)])
def test_plan_extremes_give_the_same_answer(h_q, units):
    inp = cases.small_batch([1, 640, 65, 2000, 128], s_q=1, h_q=h_q, seed=17)
    _say("plan with %d units, h_q=%d" % (units, h_q))
    out, lse, (meta, splits) = run_library(inp, num_units=units)
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, "units=%d" % units)


@pytest.mark.parametrize("s_q,h_q,units", [(4, 16, 200), (4, 8, 200), (8, 128, 40)],
                         ids=["64-row", "16-row", "1024-row"])
def test_split_partials_that_see_no_token(s_q, h_q, units):
    """Causal rows whose last split covers only tokens they may not see (a partial
    with lse = -inf, weight 0 in the combine), and a sequence shorter than s_q whose
    first new tokens see nothing at all (out = 0, lse = -inf); many units, so every
    sequence is split at its blocks."""
    inp = cases.small_batch([130, 2, 65, 200], s_q=s_q, h_q=h_q, seed=s_q * h_q + units)
    _say("masked split partials s_q=%d h_q=%d units=%d" % (s_q, h_q, units))
    out, lse, (meta, splits) = run_library(inp, num_units=units)
    assert (np.diff(splits) > 1).sum() >= 2, "the plan should split the longer sequences"
    ref_out, ref_lse = _oracle(inp)
    assert np.isneginf(ref_lse).any(), "some query should see no token"
    assert_parity(out, lse, ref_out, ref_lse, "masked partials")


@pytest.mark.parametrize("units", [1, 2, 3])
def test_wide_units_longer_than_a_table_window(units):
    """64-row kernel with a few units over sequences of 141, 79 and 2 blocks: a unit
    walks more than 64 blocks of one sequence (the copy cursor's 64-entry window of
    the block table is reloaded inside a segment and at segment changes), and split
    and unsplit sequences take both result-store paths (fp32 partials, bf16 rows)."""
    inp = cases.small_batch([9000, 5040, 100], s_q=1, h_q=64, seed=230 + units)
    _say("wide kernel, %d units over 141 + 79 + 2 blocks" % units)
    out, lse, _ = run_library(inp, num_units=units)
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, "wide units=%d" % units)


def test_large_scores_stay_finite():
    inp = cases.small_batch([150, 1000], s_q=1, h_q=16, seed=21)
    inp.q[:] = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(inp.q) * 16.0)
    _say("large scores")
    out, lse, _ = run_library(inp)
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, "large scores")


# ------------------------------------------------------------- exact properties

def test_block_table_permutation_is_bitwise_invariant():
    inp = cases.small_batch([70, 500, 64, 1], s_q=2, h_q=32, seed=23)
    _say("block permutation")
    out1, lse1, _ = run_library(inp)
    pi = np.random.default_rng(5).permutation(inp.kcache.shape[0])
    kc2 = np.empty_like(inp.kcache)
    kc2[pi] = inp.kcache
    t2 = inp.block_table.copy()
    t2[t2 >= 0] = pi[t2[t2 >= 0]]
    inp2 = wl.DecodeInputs(name="perm", q=inp.q, kcache=kc2, block_table=t2, cache_seqlens=inp.cache_seqlens,
                           s_q=inp.s_q, h_q=inp.h_q, softmax_scale=inp.softmax_scale, causal=inp.causal)
    out2, lse2, _ = run_library(inp2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_repeat_runs_are_bitwise_identical():
    inp = wl.make_workload("memory_bound")
    _say("determinism")
    dev = to_device(inp)
    a = run_library(inp, dev)
    b = run_library(inp, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_device_plan_matches_host_plan(name):
    rng = np.random.default_rng(wl.WORKLOADS[name])
    lens = wl._seqlens(name, rng)
    s_q, h_q, _ = wl._shape(name)
    _say("plan " + name)
    units = mla.mla_plan_sizes(len(lens), s_q, h_q)["num_units"]
    dmeta, dsplits = mla.mla_get_metadata(torch.from_numpy(lens).cuda(), h_q, s_q)
    hmeta, hsplits = mla.mla_get_metadata_host(lens, h_q, s_q, units)
    assert np.array_equal(dmeta.cpu().numpy(), hmeta)
    assert np.array_equal(dsplits.cpu().numpy(), hsplits)


@pytest.mark.parametrize("h_q,units", [(16, 5000 + 777), (128, 777)])
def test_device_plan_large_batch(h_q, units):
    lens = np.random.default_rng(3).integers(0, 20000, 5000).astype(np.int32)
    _say("plan B=5000 h_q=%d units=%d" % (h_q, units))
    dmeta, dsplits = mla.mla_get_metadata(torch.from_numpy(lens).cuda(), h_q, 1, num_units=units)
    hmeta, hsplits = mla.mla_get_metadata_host(lens, h_q, 1, units)
    assert np.array_equal(dmeta.cpu().numpy(), hmeta) and np.array_equal(dsplits.cpu().numpy(), hsplits)


@pytest.mark.parametrize("seed", range(6))
def test_device_plan_small_batches(seed):
    """Batches of at most 64 sequences take the planner's per-wave path; its rows equal the host planner's
    for both plan shapes, empty sequences and unit counts from the least accepted to many more than blocks."""
    rng = np.random.default_rng(500 + seed)
    for trial in range(8):
        B = 64 if trial == 0 else int(rng.integers(1, 65))
        lens = rng.integers(0, 9000, B).astype(np.int32)
        lens[rng.random(B) < 0.15] = 0
        s_q, h_q = [(1, 16), (2, 16), (1, 64), (1, 128), (3, 16), (2, 64)][(seed + trial) % 6]
        by_sequence = (s_q * h_q) % 64 != 0
        units = int(rng.choice([1, 2, 7, 64, 256, 999])) + (B if by_sequence else 0)
        _say("small plan B=%d s_q=%d h_q=%d units=%d" % (B, s_q, h_q, units))
        dmeta, dsplits = mla.mla_get_metadata(torch.from_numpy(lens).cuda(), h_q, s_q, num_units=units)
        hmeta, hsplits = mla.mla_get_metadata_host(lens, h_q, s_q, units)
        assert np.array_equal(dmeta.cpu().numpy(), hmeta), (B, s_q, h_q, units)
        assert np.array_equal(dsplits.cpu().numpy(), hsplits), (B, s_q, h_q, units)


# ------------------------------------------------------------- graph capture

@pytest.mark.parametrize("lens,s_q,h_q", [([700, 65, 3000, 1], 1, 16), ([300, 2000, 64], 2, 128)])
def test_graph_replays_match_eager(lens, s_q, h_q):
    """The plan + decode captured in a HIP graph (as the benchmark times it) gives, on every
    replay, exactly the eager result; eager work and synchronisations run between replays."""
    _say("graph capture lens=%s s_q=%d h_q=%d" % (lens, s_q, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=sum(lens) + 7)
    dev = to_device(inp)
    B = len(lens)
    units = mla.mla_plan_sizes(B, s_q, h_q)["num_units"]
    meta = torch.empty((units, mla.META_INTS), dtype=torch.int32, device="cuda:0")
    splits = torch.empty((B + 1,), dtype=torch.int32, device="cuda:0")
    out = torch.empty((B, s_q, h_q, mla.D_V), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device="cuda:0")
    ws = torch.empty((mla.workspace_bytes(B, s_q, h_q, units),), dtype=torch.uint8, device="cuda:0")

    def run():
        mla.mla_get_metadata(dev["cache_seqlens"], h_q, s_q, num_units=units, tile_meta=meta, num_splits=splits)
        mla.mla_decode_fwd(dev["q"], dev["kcache"], dev["block_table"], dev["cache_seqlens"], inp.softmax_scale,
                           meta, splits, causal=inp.causal, out=out, lse=lse, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        run()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        meta.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "replay %d differs" % rep
        run()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), "eager run after replay %d differs" % rep
    ref_out, ref_lse = _oracle(inp)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, "graph")
