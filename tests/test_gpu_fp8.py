"""GPU parity of the FP8 latent cache: the quantizing append bit-exact against the
CPU quantizer (codes and scales), the FP8 decode against the FP8 CPU oracle
(tiny, memory-bound at full size, edge shapes, NaN in every row no query may
read, several head groups, two causal new tokens), and an append-then-decode
step, all through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
import workloads as wl
from oracle import fp8
from tests import cases
from tests.gpu_util import assert_parity, rel_rms

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def run(inp, codes, scales, num_units=None):
    dev_lens = torch.from_numpy(inp.cache_seqlens).cuda()
    meta, splits = mla.mla_get_metadata_fp8(dev_lens, inp.h_q, inp.s_q, num_units=num_units)
    out, lse = mla.mla_decode_fp8_fwd(bf16_dev(inp.q), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                      torch.from_numpy(inp.block_table).cuda(), dev_lens, inp.softmax_scale, meta,
                                      splits, causal=inp.causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def ref(inp, codes, scales):
    return oracle.mla_decode_fp8(inp.q, codes, scales, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                                 inp.causal)


def clean_rows(inp):
    """Rows the quantizer may see: NaN-poisoned rows become zeros before quantizing."""
    k = inp.kcache.copy()
    k[np.all(k == wl.BF16_NAN, axis=-1)] = 0
    return k


@pytest.mark.parametrize("name", ["tiny", "memory_bound"])
def test_fp8_workloads(name):
    _say("fp8 workload " + name)
    inp = wl.make_workload(name, poison=True)
    codes, scales = fp8.quantize_rows(clean_rows(inp))
    bad = np.all(inp.kcache == wl.BF16_NAN, axis=-1)
    codes[bad] = 0x7F
    scales[bad] = np.nan
    out, lse = run(inp, codes, scales)
    ro, rl = ref(inp, codes, scales)
    assert_parity(out, lse, ro, rl, name)
    print("rel rms %.2e" % rel_rms(out, ro))


EDGE = [([64, 200, 1], 1, 16), ([31, 33, 95, 97], 2, 16), ([1, 2, 3], 4, 16), ([0, 130, 0], 1, 16),
        ([300, 64], 2, 64), ([129, 1000], 1, 128), ([5000], 1, 16), ([100, 257], 3, 32)]


@pytest.mark.parametrize("lens,s_q,h_q", EDGE)
def test_fp8_edge_shapes(lens, s_q, h_q):
    _say("fp8 edge lens=%s s_q=%d h_q=%d" % (lens, s_q, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=sum(lens) + 17 * s_q + h_q)
    codes, scales = fp8.quantize_rows(clean_rows(inp))
    bad = np.all(inp.kcache == wl.BF16_NAN, axis=-1)
    codes[bad] = 0x7F
    scales[bad] = np.nan
    out, lse = run(inp, codes, scales)
    ro, rl = ref(inp, codes, scales)
    assert_parity(out, lse, ro, rl, "fp8 %s" % (lens,))


WIDE = [([5, 70, 1, 0, 129, 64, 3], 1, 64, True), ([1, 2, 200], 4, 16, True), ([700, 33], 2, 32, True),
        ([64, 2048], 1, 128, False), ([0, 0, 65], 1, 64, True), ([3000, 17, 400, 1], 2, 64, True)]


@pytest.mark.parametrize("lens,s_q,h_q,causal", WIDE)
def test_fp8_wide_shapes(lens, s_q, h_q, causal):
    """s_q * h_q a multiple of 64: the 64-row kernel; units span several short sequences,
    lengths below s_q, empty sequences, non-causal."""
    _say("fp8 wide lens=%s s_q=%d h_q=%d causal=%d" % (lens, s_q, h_q, causal))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=7 * sum(lens) + h_q, causal=causal)
    codes, scales = fp8.quantize_rows(clean_rows(inp))
    bad = np.all(inp.kcache == wl.BF16_NAN, axis=-1)
    codes[bad] = 0x7F
    scales[bad] = np.nan
    out, lse = run(inp, codes, scales)
    ro, rl = ref(inp, codes, scales)
    assert_parity(out, lse, ro, rl, "fp8 wide %s" % (lens,))


@pytest.mark.parametrize("units", [3, 7, 300])
def test_fp8_wide_plan_extremes(units):
    _say("fp8 wide units=%d" % units)
    inp = cases.small_batch([900, 64, 2000, 5, 130], s_q=1, h_q=64, seed=units + 1)
    codes, scales = fp8.quantize_rows(clean_rows(inp))
    out, lse = run(inp, codes, scales, num_units=units)
    ro, rl = ref(inp, codes, scales)
    assert_parity(out, lse, ro, rl, "wide units %d" % units)


@pytest.mark.parametrize("units", [1, 2])
def test_fp8_wide_units_longer_than_a_table_window(units):
    """The FP8 64-row kernel with units that walk more than 64 blocks of one sequence
    (block-table window reloads inside a segment and at segment changes)."""
    _say("fp8 wide, %d units over 141 + 79 + 2 blocks" % units)
    inp = cases.small_batch([9000, 5040, 100], s_q=1, h_q=64, seed=240 + units)
    codes, scales = fp8.quantize_rows(clean_rows(inp))
    out, lse = run(inp, codes, scales, num_units=units)
    ro, rl = ref(inp, codes, scales)
    assert_parity(out, lse, ro, rl, "fp8 wide units %d" % units)


@pytest.mark.parametrize("units", [17, 40, 900])
def test_fp8_plan_extremes(units):
    _say("fp8 units=%d" % units)
    inp = cases.small_batch([900, 64, 2000, 5], s_q=1, h_q=16, seed=units)
    codes, scales = fp8.quantize_rows(clean_rows(inp))
    out, lse = run(inp, codes, scales, num_units=units)
    ro, rl = ref(inp, codes, scales)
    assert_parity(out, lse, ro, rl, "units %d" % units)


@pytest.mark.parametrize("lens,s_new", [([64, 200, 1], 1), ([300, 70], 64), ([129, 1, 3000], 100)])
def test_fp8_append_bit_exact(lens, s_new):
    _say("fp8 append lens=%s s_new=%d" % (lens, s_new))
    rng = np.random.default_rng(sum(lens) + s_new)
    inp = wl.build_inputs(np.asarray(lens, np.int32), 1, 16, rng, name="a", causal=True, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    new = wl.f32_to_bf16_bits((rng.standard_normal((len(lens), s_new, 576)) *
                               rng.uniform(1e-3, 1e3, (len(lens), s_new, 1))).astype(np.float32))
    new[0, 0] = 0                                           # a zero row
    rc, rs = fp8.append_rows_fp8(codes, scales, inp.block_table, inp.cache_seqlens, new)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    mla.mla_append_kv_fp8(dc, ds, torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.cache_seqlens).cuda(),
                          bf16_dev(new))
    torch.cuda.synchronize()
    assert np.array_equal(dc.cpu().numpy(), rc)
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_fp8_append_then_decode():
    """A decode step on the FP8 cache: the new rows are quantized by the GPU append and
    decoded by the FP8 kernel; the oracle quantizes and decodes on the CPU."""
    _say("fp8 append then decode")
    inp = cases.small_batch([500, 70, 129], s_q=2, h_q=16, seed=9)
    base = clean_rows(inp)
    codes, scales = fp8.quantize_rows(base)
    rng = np.random.default_rng(3)
    new = wl.f32_to_bf16_bits(rng.standard_normal((3, 2, 576)).astype(np.float32))
    rc, rs = fp8.append_rows_fp8(codes, scales, inp.block_table, inp.cache_seqlens, new)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    lens = torch.from_numpy(inp.cache_seqlens).cuda()
    table = torch.from_numpy(inp.block_table).cuda()
    mla.mla_append_kv_fp8(dc, ds, table, lens, bf16_dev(new))
    meta, splits = mla.mla_get_metadata_fp8(lens, inp.h_q, inp.s_q)
    out, lse = mla.mla_decode_fp8_fwd(bf16_dev(inp.q), dc, ds, table, lens, inp.softmax_scale, meta, splits,
                                      causal=True)
    torch.cuda.synchronize()
    ro, rl = ref(inp, rc, rs)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "append+decode")


def test_fp8_mixed_sampled_rows():
    """The mixed workload (s_q=2, h_q=128, causal, lengths 256-16384) on the FP8 cache; sampled sequences."""
    _say("fp8 mixed sampled")
    inp = wl.make_workload("mixed", poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    out, lse = run(inp, codes, scales)
    lens = inp.cache_seqlens
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5})
    for b in pick:
        sub = wl.subset(inp, [b])
        ro, rl = ref(sub, codes, scales)
        assert_parity(out[[b]], lse[[b]], ro, rl, "mixed row %d" % b)


def test_fp8_compute_bound_sampled_rows():
    """The compute-bound workload (h_q=128, eight head groups) on the FP8 cache; sampled sequences."""
    _say("fp8 compute_bound sampled")
    inp = wl.make_workload("compute_bound", poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    out, lse = run(inp, codes, scales)
    rng = np.random.default_rng(1)
    for b in rng.choice(inp.batch, size=2, replace=False):
        sub = wl.subset(inp, [b])
        ro, rl = ref(sub, codes, scales)
        assert_parity(out[[b]], lse[[b]], ro, rl, "compute_bound row %d" % b)
