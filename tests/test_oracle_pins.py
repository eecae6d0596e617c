"""Pins for the CPU oracle: what the pages and the mathematics fix, independent of the oracle's code.

Each check takes a decode callable (the oracle, or a copy of it with a planted
mistake) and raises AssertionError on a mismatch:
  * golden: hand-derived cases (tests/golden/closed_form_cases.json);
  * library: torch's scaled_dot_product_attention and logsumexp in float64 on
    densely gathered rows (a library routine, MQA-style one shared K/V head);
  * single token: one visible token returns its V row, lse = its scaled score;
  * equal scores: q = 0 returns the mean of the visible V rows, lse = ln(count);
  * permutation: relabelling physical blocks (and the table with them) changes nothing;
  * causal prefix: query i of s_q new tokens equals a one-token decode over the first L-s_q+1+i tokens;
  * two-part merge: attention over a split token range, merged by log-sum-exp, equals the whole;
  * stability: large scores stay finite and approach the arg-max row;
  * poison: NaN in rows nobody may read changes nothing.
The mutation test plants plausible mistakes in a copy of the oracle source and
requires each to fail at least one check.
"""
from __future__ import annotations

import math
import os
import shutil
import tempfile
from pathlib import Path

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl
from tests import cases


def _dec(lib):
    def run(inp, **kw):
        return oracle.mla_decode(inp.q, inp.kcache, inp.block_table, inp.cache_seqlens,
                                 kw.get("scale", inp.softmax_scale), inp.causal, nthreads=4, lib=lib)
    return run


# ---------------------------------------------------------------- checks

def check_golden(dec):
    for inp, exp_out, exp_lse in cases.golden_cases():
        out, lse = dec(inp)
        assert np.allclose(out, exp_out, rtol=0, atol=1e-9), inp.name
        assert np.allclose(lse, exp_lse, rtol=0, atol=1e-9, equal_nan=False), (inp.name, lse, exp_lse)


def _library_reference(inp):
    B = inp.batch
    out = np.zeros((B, inp.s_q, inp.h_q, wl.D_V))
    lse = np.full((B, inp.s_q, inp.h_q), -np.inf)
    q = torch.from_numpy(wl.bf16_bits_to_f32(inp.q).astype(np.float64))
    for b in range(B):
        L = int(inp.cache_seqlens[b])
        K = torch.from_numpy(cases.gather_dense_k(inp, b))
        V = K[:, :wl.D_V]
        i = torch.arange(inp.s_q)[:, None]
        t = torch.arange(L)[None, :]
        mask = (t <= L - inp.s_q + i) if inp.causal else torch.ones(inp.s_q, L, dtype=torch.bool)
        qb = q[b].transpose(0, 1)                      # [h, s_q, d]
        ob = F.scaled_dot_product_attention(qb[None], K.expand(inp.h_q, L, -1)[None],
                                            V.expand(inp.h_q, L, -1)[None],
                                            attn_mask=mask, scale=inp.softmax_scale)[0]
        sc = torch.matmul(qb, K.T) * inp.softmax_scale
        lb = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)
        vis = mask.any(dim=-1)
        ob = torch.where(vis[None, :, None], ob, torch.zeros_like(ob))
        out[b] = ob.transpose(0, 1).numpy()
        lse[b] = lb.transpose(0, 1).numpy()
    return out, lse


def check_library(dec):
    for lens, s_q, h_q, seed in [([1, 63, 64, 65, 130], 1, 4, 1), ([200, 3, 129], 2, 8, 2),
                                 ([64, 200], 1, 16, 3), ([7, 70], 3, 2, 4)]:
        inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=seed)
        out, lse = dec(inp)
        ro, rl = _library_reference(inp)
        assert np.allclose(out, ro, rtol=1e-10, atol=1e-12), (lens, s_q, float(np.abs(out - ro).max()))
        assert np.allclose(lse, rl, rtol=1e-12, atol=1e-12), (lens, s_q)


def check_single_token(dec):
    inp = cases.small_batch([1, 1, 1], s_q=1, h_q=8, seed=5)
    out, lse = dec(inp)
    q = wl.bf16_bits_to_f32(inp.q).astype(np.float64)
    for b in range(inp.batch):
        k0 = wl.bf16_bits_to_f32(inp.kcache[inp.block_table[b, 0], 0]).astype(np.float64)
        for h in range(inp.h_q):
            assert np.array_equal(out[b, 0, h], k0[:wl.D_V]), b
            assert abs(lse[b, 0, h] - inp.softmax_scale * float(q[b, 0, h] @ k0)) < 1e-10


def check_equal_scores(dec):
    for lens, s_q in [([5, 64, 150], 1), ([9, 66], 2)]:
        inp = cases.small_batch(lens, s_q=s_q, h_q=4, seed=6)
        inp.q[:] = 0
        out, lse = dec(inp)
        vis = wl.visible_tokens(inp.cache_seqlens, s_q, inp.causal)
        for b in range(inp.batch):
            K = cases.gather_dense_k(inp, b)
            for i in range(s_q):
                n = int(vis[b, i])
                mean = K[:n, :wl.D_V].mean(axis=0)
                for h in range(inp.h_q):
                    assert np.allclose(out[b, i, h], mean, rtol=1e-12, atol=1e-13), (b, i)
                    assert abs(lse[b, i, h] - math.log(n)) < 1e-12


def check_permutation(dec):
    inp = cases.small_batch([70, 200, 64], s_q=2, h_q=4, seed=7)
    out, lse = dec(inp)
    rng = np.random.default_rng(70)
    nblocks = inp.kcache.shape[0]
    pi = rng.permutation(nblocks)                 # new id of old block p is pi[p]
    kc2 = np.empty_like(inp.kcache)
    kc2[pi] = inp.kcache
    t2 = inp.block_table.copy()
    used = t2 >= 0
    t2[used] = pi[t2[used]]
    inp2 = wl.DecodeInputs(name="perm", q=inp.q, kcache=kc2, block_table=t2,
                           cache_seqlens=inp.cache_seqlens, s_q=inp.s_q, h_q=inp.h_q,
                           softmax_scale=inp.softmax_scale, causal=inp.causal)
    out2, lse2 = dec(inp2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def check_causal_prefix(dec):
    lens = [67, 130, 5]
    s_q = 3
    inp = cases.small_batch(lens, s_q=s_q, h_q=4, seed=8)
    out, lse = dec(inp)
    for i in range(s_q):
        lens_i = np.array([L - s_q + 1 + i for L in lens], dtype=np.int32)
        one = wl.DecodeInputs(name="prefix", q=np.ascontiguousarray(inp.q[:, i:i + 1]), kcache=inp.kcache,
                              block_table=inp.block_table, cache_seqlens=lens_i, s_q=1, h_q=inp.h_q,
                              softmax_scale=inp.softmax_scale, causal=True)
        o1, l1 = dec(one)
        assert np.allclose(out[:, i], o1[:, 0], rtol=1e-13, atol=1e-14), i
        assert np.allclose(lse[:, i], l1[:, 0], rtol=1e-13, atol=1e-14), i


def check_two_part_merge(dec):
    # one sequence of 5 blocks (300 tokens) split after 2 blocks into two sequences
    inp = cases.small_batch([300], s_q=1, h_q=8, seed=9)
    whole_o, whole_l = dec(inp)
    tab = inp.block_table[0]
    parts = wl.DecodeInputs(name="parts", q=np.concatenate([inp.q, inp.q]), kcache=inp.kcache,
                            block_table=np.stack([np.concatenate([tab[:2], [-1, -1, -1]]),
                                                  np.concatenate([tab[2:], [-1, -1]])]).astype(np.int32),
                            cache_seqlens=np.array([128, 172], dtype=np.int32), s_q=1, h_q=inp.h_q,
                            softmax_scale=inp.softmax_scale, causal=False)
    po, pl = dec(parts)
    lse = np.logaddexp(pl[0], pl[1])
    out = np.exp(pl[0] - lse)[..., None] * po[0] + np.exp(pl[1] - lse)[..., None] * po[1]
    assert np.allclose(lse, whole_l[0], rtol=1e-13, atol=1e-13)
    assert np.allclose(out, whole_o[0], rtol=1e-11, atol=1e-13)


def check_stability(dec):
    for scale in (1.0 / math.sqrt(192.0), 1.0):
        _check_stability_at(dec, scale)


def _check_stability_at(dec, scale):
    # scores reach hundreds (scale 1/sqrt(192)) or thousands (scale 1), far past exp's range
    inp = cases.small_batch([150, 64], s_q=1, h_q=4, seed=10, scale=scale)
    inp.q[:] = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(inp.q) * 64.0)
    out, lse = dec(inp)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    q = wl.bf16_bits_to_f32(inp.q).astype(np.float64)
    for b in range(inp.batch):
        K = cases.gather_dense_k(inp, b)
        s = inp.softmax_scale * (q[b, 0] @ K.T)           # [h, L]
        top = np.argmax(s, axis=1)
        gap = np.sort(s, axis=1)[:, -1] - np.sort(s, axis=1)[:, -2]
        for h in range(inp.h_q):
            assert lse[b, 0, h] >= s[h, top[h]] - 1e-9
            assert lse[b, 0, h] <= s[h, top[h]] + math.log(K.shape[0]) + 1e-9
            if gap[h] > 40:
                assert np.allclose(out[b, 0, h], K[top[h], :wl.D_V], rtol=1e-9, atol=1e-9)


def check_poison(dec):
    clean = cases.small_batch([65, 130, 1], s_q=2, h_q=4, seed=11, poison=False)
    dirty = cases.small_batch([65, 130, 1], s_q=2, h_q=4, seed=11, poison=True)
    assert not np.array_equal(clean.kcache, dirty.kcache)
    o1, l1 = dec(clean)
    o2, l2 = dec(dirty)
    assert np.isfinite(o2).all()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


CHECKS = [check_golden, check_library, check_single_token, check_equal_scores, check_permutation,
          check_causal_prefix, check_two_part_merge, check_stability, check_poison]


@pytest.fixture(scope="module")
def real_oracle():
    return _dec(oracle.load())


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(real_oracle, check):
    check(real_oracle)


def test_oracle_rejects_bad_arguments():
    lib = oracle.load()
    assert lib.mla_oracle_decode(None, None, None, None, 1, 1, 1, 1, 576, 512, 64, 1.0, 1, None, None, 1) == -1
    assert lib.mla_oracle_decode(None, None, None, None, 1, 0, 1, 1, 576, 512, 64, 1.0, 1, None, None, 1) == -1


def test_oracle_thread_count_does_not_change_results():
    inp = cases.small_batch([100, 37, 64], s_q=2, h_q=8, seed=12)
    a = oracle.decode_inputs(inp, nthreads=1)
    b = oracle.decode_inputs(inp, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "rope_columns_dropped": ("for (int d = 0; d < a->d_qk; ++d) dot +=",
                             "for (int d = 0; d < a->d_v; ++d) dot +="),
    "scale_dropped": ("score[t] = a->scale * dot;", "score[t] = dot;"),
    "causal_off_by_one": ("long visible = a->causal ? L - (a->s_q - 1 - i) : L;",
                          "long visible = a->causal ? L - (a->s_q - i) : L;"),
    "causal_reversed": ("long visible = a->causal ? L - (a->s_q - 1 - i) : L;",
                        "long visible = a->causal ? L - i : L;"),
    "block_table_ignored": ("long phys = a->block_table[(long)b * a->max_blocks + j];",
                            "long phys = a->block_table[(long)b * a->max_blocks] + j;"),
    "page_row_index": ("long r = t % a->page;", "long r = (t + 1) % a->page;"),
    "lse_without_max": ("a->lse[row] = m + log(denom);", "a->lse[row] = log(denom);"),
    "lse_log2": ("a->lse[row] = m + log(denom);", "a->lse[row] = m + log2(denom);"),
    "value_from_last_columns": ("out[c] += w * bf16_value(v[c]);",
                                "out[c] += w * bf16_value(v[c + a->d_qk - a->d_v]);"),
    "not_normalised": ("double w = exp(score[t] - m) / denom;", "double w = exp(score[t] - m);"),
    "denominator_unshifted": ("denom += exp(score[t] - m);", "denom += exp(score[t]);"),
    "first_token_value_dropped": ("for (long t = 0; t < visible; ++t) {\n        const uint16_t* v",
                                  "for (long t = 1; t < visible; ++t) {\n        const uint16_t* v"),
    "row_layout_transposed": ("const long row = ((long)b * a->s_q + i) * a->h_q + h;",
                              "const long row = ((long)b * a->h_q + h) * a->s_q + i;"),
    "last_token_unseen": ("for (long t = 0; t < visible; ++t) {\n        const uint16_t* k",
                          "for (long t = 0; t + 1 < visible; ++t) {\n        const uint16_t* k"),
    "max_from_first_score_only": ("if (score[t] > m) m = score[t];", "if (0) m = score[t];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = oracle._SRC.read_text()
    assert src.count(old) == 1, "mutation anchor not found: " + name
    tmp = Path(tempfile.mkdtemp(prefix="oracle_mutant_"))
    try:
        msrc = tmp / "mutant.c"
        msrc.write_text(src.replace(old, new))
        lib = oracle.load(oracle.build(force=True, src=msrc, out=tmp / "libmutant.so"))
        dec = _dec(lib)
        failed = []
        for check in CHECKS:
            try:
                with np.errstate(all="ignore"):
                    check(dec)
            except (AssertionError, RuntimeError, ValueError, IndexError):
                failed.append(check.__name__)
        assert failed, "planted mistake %s passed every pin" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
