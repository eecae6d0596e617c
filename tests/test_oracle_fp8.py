"""Pins of the FP8 cache oracle (oracle/mla_oracle_fp8.c, oracle/fp8.py), CPU only.

  * format: all 256 E4M3 codes decode (C and Python) to torch's float8_e4m3fn values;
  * rounding: the quantizer's float32 -> E4M3 step equals torch's float8_e4m3fn cast
    for every in-range value tried (random values, every midpoint between codes);
  * quantizer: the row maximum lands exactly on +-448, no other code is nearer to any
    scaled value, zero rows give scale 0;
  * decode: with power-of-two scales (decoded values exact in bf16) the FP8 oracle equals
    bitwise the bf16 oracle on a cache holding the decoded values; with any scales it
    equals torch's float64 attention over the decoded rows; NaN codes in rows nobody
    may read change nothing;
  * append: the FP8 append writes exactly the quantized new rows where the bf16 append
    writes the new rows;
  * planted mistakes in a copy of the C source each fail a check.
"""
from __future__ import annotations

import math
import shutil
import tempfile
from pathlib import Path

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl
from oracle import append as app
from oracle import fp8


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_code_values_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_e4m3(codes)
    mine = fp8.e4m3_table()
    lib = oracle.load()
    c = np.array([lib.mla_oracle_e4m3_value(int(k)) for k in range(256)])
    for v in (mine, c):
        same = (v == ref) | (np.isnan(v) & np.isnan(ref))
        assert same.all(), np.nonzero(~same)


def test_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    vals = fp8.e4m3_table()
    pos = np.sort(vals[:127])
    mids = (pos[1:] + pos[:-1]) / 2                    # exact ties between neighbouring codes
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** -6,
                        mids, -mids, pos, -pos, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    mine = fp8.round_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    same = (mine == ref) | ((vals[mine] == 0) & (vals[ref] == 0))
    assert same.all(), x[~same][:10]


def test_quantizer_properties():
    rng = np.random.default_rng(1)
    rows = wl.f32_to_bf16_bits((rng.standard_normal((300, 576)) * rng.uniform(1e-3, 1e3, (300, 1))).astype(np.float32))
    rows[7] = 0
    codes, scales = fp8.quantize_rows(rows)
    x = wl.bf16_bits_to_f32(rows).astype(np.float64)
    vals = fp8.e4m3_table()
    assert scales[7] == 0 and (codes[7] == 0).all()
    for r in range(300):
        if r == 7:
            continue
        k = int(np.argmax(np.abs(x[r])))
        assert abs(vals[codes[r, k]]) == 448.0
        y = (x[r].astype(np.float32) * np.float32(np.float32(448) / np.float32(np.abs(x[r]).max()))).astype(np.float64)
        d = np.abs(vals[codes[r]] - y)
        dist = np.abs(vals[None, :127] * np.sign(y)[:, None] - y[:, None])
        assert (d <= dist.min(axis=1) + 0).all()
        assert scales[r] == np.float32(np.float32(np.abs(x[r]).max()) / np.float32(448))


def fp8_case(lens, s_q, h_q, seed, pow2=False, poison=True):
    rng = np.random.default_rng(seed)
    inp = wl.build_inputs(np.asarray(lens, np.int32), s_q, h_q, rng, name="fp8", causal=True, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    if pow2:
        scales = (2.0 ** np.round(np.log2(np.maximum(scales, 1e-30)))).astype(np.float32)
    if poison:
        nb = (np.asarray(lens) + 63) // 64
        used = np.zeros(codes.shape[0], dtype=bool)
        for b, n in enumerate(nb):
            used[inp.block_table[b, :n]] = True
            tail = int(lens[b]) - (int(n) - 1) * 64
            if tail < 64:
                codes[inp.block_table[b, n - 1], tail:] = 0x7F
                scales[inp.block_table[b, n - 1], tail:] = np.nan
        codes[~used] = 0x7F
        scales[~used] = np.nan
    return inp, codes, scales


def _run(lib):
    def run(inp, codes, scales):
        return oracle.mla_decode_fp8(inp.q, codes, scales, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                                     inp.causal, nthreads=4, lib=lib)
    return run


def check_bf16_equivalence(run):
    inp, codes, scales = fp8_case([64, 200, 7], 2, 16, seed=3, pow2=True, poison=False)
    o, l = run(inp, codes, scales)
    deq = fp8.dequantize(codes, scales).astype(np.float32)
    bf = wl.f32_to_bf16_bits(deq)
    assert np.array_equal(wl.bf16_bits_to_f32(bf).astype(np.float64), fp8.dequantize(codes, scales))
    ro, rl = oracle.mla_decode(inp.q, bf, inp.block_table, inp.cache_seqlens, inp.softmax_scale, inp.causal)
    assert np.array_equal(o, ro) and np.array_equal(l, rl)


def check_library(run):
    inp, codes, scales = fp8_case([130, 70], 2, 8, seed=4)
    o, l = run(inp, codes, scales)
    for b, L in enumerate(inp.cache_seqlens):
        rows = []
        for t in range(int(L)):
            blk = inp.block_table[b, t // 64]
            rows.append(fp8.dequantize(codes[blk, t % 64][None], scales[blk, t % 64][None])[0])
        K = torch.from_numpy(np.array(rows))
        for i in range(inp.s_q):
            n = int(L) - (inp.s_q - 1 - i)
            Q = torch.from_numpy(wl.bf16_bits_to_f32(inp.q[b, i]).astype(np.float64))
            ref = F.scaled_dot_product_attention(Q[None, :, None, :].transpose(1, 2), K[None, None, :n],
                                                 K[None, None, :n, :512], scale=inp.softmax_scale)[0, 0]
            rl = torch.logsumexp(inp.softmax_scale * (Q @ K[:n].T), dim=-1)
            assert np.allclose(o[b, i], ref.numpy(), rtol=1e-9, atol=1e-12)
            assert np.allclose(l[b, i], rl.numpy(), rtol=1e-12, atol=1e-12)


def check_poison(run):
    inp, codes, scales = fp8_case([100, 300], 1, 8, seed=5, poison=True)
    _, c2, s2 = fp8_case([100, 300], 1, 8, seed=5, poison=False)
    o1, l1 = run(inp, codes, scales)
    o2, l2 = run(inp, c2, s2)
    assert np.isfinite(o1).all() and np.array_equal(o1, o2) and np.array_equal(l1, l2)


CHECKS = [check_bf16_equivalence, check_library, check_poison]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_fp8_oracle_pin(check):
    check(_run(oracle.load()))


def test_fp8_append_matches_bf16_append():
    rng = np.random.default_rng(6)
    lens = np.array([70, 5, 200], np.int32)
    inp = wl.build_inputs(lens, 1, 8, rng, name="a", causal=True, poison=False)
    codes, scales = fp8.quantize_rows(inp.kcache)
    new = wl.f32_to_bf16_bits(rng.standard_normal((3, 9, 576)).astype(np.float32))
    c2, s2 = fp8.append_rows_fp8(codes, scales, inp.block_table, lens, new)
    bf = app.append_rows(inp.kcache, inp.block_table, lens, new)
    changed = np.any(bf != inp.kcache, axis=-1)
    qc, qs = fp8.quantize_rows(bf)
    assert np.array_equal(c2[changed], qc[changed]) and np.array_equal(s2[changed], qs[changed])
    assert np.array_equal(c2[~changed], codes[~changed]) and np.array_equal(s2[~changed], scales[~changed])
    assert changed.sum() == sum(min(9, int(n)) for n in lens)


MUTANTS = {
    "subnormal_exponent": ("if (expo == 0) v = ldexp((double)mant / 8.0, -6);",
                           "if (expo == 0) v = ldexp((double)mant / 8.0, -7);"),
    "exponent_bias": ("else v = ldexp(1.0 + (double)mant / 8.0, expo - 7);",
                      "else v = ldexp(1.0 + (double)mant / 8.0, expo - 8);"),
    "sign_ignored": ("return sign ? -v : v;", "return v;"),
    "key_scale_dropped": ("dot += q_value(qrow[d]) * (mla_oracle_e4m3_value(k[d]) * ks);",
                          "dot += q_value(qrow[d]) * mla_oracle_e4m3_value(k[d]);"),
    "value_scale_dropped": ("out[c] += w * (mla_oracle_e4m3_value(v[c]) * vs);",
                            "out[c] += w * mla_oracle_e4m3_value(v[c]);"),
    "value_scale_of_first_row": ("const double vs = (double)a->scales[phys];",
                                 "const double vs = (double)a->scales[(long)a->block_table[(long)b * a->max_blocks] * a->page];"),
    "causal_off_by_one": ("const long n = a->causal ? L - (a->s_q - 1 - i) : L;",
                          "const long n = a->causal ? L - (a->s_q - i) : L;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = oracle._SRC_FP8.read_text()
    assert src.count(old) == 1, "mutation anchor not found: " + name
    tmp = Path(tempfile.mkdtemp(prefix="fp8_mutant_"))
    try:
        msrc = tmp / "mutant.c"
        msrc.write_text(src.replace(old, new))
        lib = oracle.load(oracle.build(force=True, src=[oracle._SRC, msrc], out=tmp / "libmutant.so"))
        failed = []
        for check in CHECKS + [lambda run: test_code_values_via(lib)]:
            try:
                with np.errstate(all="ignore"):
                    check(_run(lib))
            except (AssertionError, RuntimeError, ValueError, IndexError):
                failed.append(getattr(check, "__name__", "codes"))
        assert failed, "planted mistake %s passed every pin" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_code_values_via(lib):
    ref = torch_e4m3(np.arange(256, dtype=np.uint8))
    c = np.array([lib.mla_oracle_e4m3_value(int(k)) for k in range(256)])
    assert ((c == ref) | (np.isnan(c) & np.isnan(ref))).all()


@pytest.fixture
def lib():
    return oracle.load()
