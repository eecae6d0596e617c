"""Pins of the sparse (top-k index) decode oracle, oracle/mla_oracle_sparse.c (CPU only).

Each check takes a sparse-decode callable and raises AssertionError on a mismatch:
  * dense: the full sorted list [0, L) gives bitwise the dense oracle's non-causal
    result (an independently written and separately pinned file);
  * library: torch's scaled_dot_product_attention / logsumexp in float64 over the
    listed rows gathered densely (repeats included);
  * order: a permuted list gives the same result to 1e-12;
  * padding: entries < 0 anywhere in the list change nothing (bitwise);
  * counts: only the first counts[.] entries are read (the rest may be anything);
  * single entry: out is its V row and lse its scaled score;
  * empty: a list with no valid entry gives out = 0, lse = -inf.
Planted mistakes in a copy of the C source must each fail at least one check.
"""
from __future__ import annotations

import shutil
import tempfile
from pathlib import Path

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl


def sparse_case(lens, s_q, h_q, topk, seed, dup=False):
    rng = np.random.default_rng(seed)
    inp = wl.build_inputs(np.asarray(lens, dtype=np.int32), s_q, h_q, rng, name="sparse", causal=False,
                          poison=True)
    B = len(lens)
    idx = np.full((B, s_q, topk), -1, dtype=np.int32)
    counts = np.zeros((B * s_q,), dtype=np.int32)
    for b in range(B):
        for i in range(s_q):
            n = min(topk, int(lens[b]))
            pick = rng.choice(int(lens[b]), size=n, replace=False) if n else np.zeros(0, np.int64)
            if dup and n >= 2:
                pick[1] = pick[0]
            k = int(rng.integers(max(0, n - 3), n + 1)) if n else 0     # some lists shorter than topk
            idx[b, i, :k] = pick[:k]
            counts[b * s_q + i] = k
    return inp, idx, counts


def _run(lib):
    def run(inp, idx, counts):
        return oracle.mla_decode_sparse(inp.q, inp.kcache, inp.block_table, idx, counts, inp.softmax_scale,
                                        nthreads=4, lib=lib)
    return run


CASES = [([64, 200, 5], 1, 16, 32), ([130, 70], 2, 16, 100), ([300], 3, 8, 300), ([1, 2, 40], 1, 4, 8)]


def gather_rows(inp, b, toks):
    rows = []
    for t in toks:
        rows.append(inp.kcache[inp.block_table[b, t // 64], t % 64])
    return wl.bf16_bits_to_f32(np.array(rows, dtype=np.uint16).reshape(len(toks), -1)).astype(np.float64)


def check_dense(run):
    inp = wl.make_workload("tiny", poison=True)
    B = inp.batch
    topk = int(inp.cache_seqlens.max())
    idx = np.full((B, 1, topk), -1, dtype=np.int32)
    cnt = np.zeros((B,), dtype=np.int32)
    for b in range(B):
        L = int(inp.cache_seqlens[b])
        idx[b, 0, :L] = np.arange(L)
        cnt[b] = L
    o, l = run(inp, idx, cnt)
    ro, rl = oracle.mla_decode(inp.q, inp.kcache, inp.block_table, inp.cache_seqlens, inp.softmax_scale, False)
    assert np.array_equal(o, ro) and np.array_equal(l, rl)


def check_library(run):
    for (lens, s_q, h_q, topk), seed in zip(CASES, range(4)):
        inp, idx, cnt = sparse_case(lens, s_q, h_q, topk, seed, dup=(seed % 2 == 0))
        o, l = run(inp, idx, cnt)
        for b in range(len(lens)):
            for i in range(s_q):
                toks = [int(t) for t in idx[b, i, :cnt[b * s_q + i]] if t >= 0]
                if not toks:
                    assert (o[b, i] == 0).all() and np.isneginf(l[b, i]).all()
                    continue
                K = torch.from_numpy(gather_rows(inp, b, toks))
                Q = torch.from_numpy(wl.bf16_bits_to_f32(inp.q[b, i]).astype(np.float64))
                ref = F.scaled_dot_product_attention(Q[None, :, None, :].transpose(1, 2),
                                                     K[None, None, :, :], K[None, None, :, :512],
                                                     scale=inp.softmax_scale)[0, 0]
                rl = torch.logsumexp(inp.softmax_scale * (Q @ K.T), dim=-1)
                assert np.allclose(o[b, i], ref.numpy(), rtol=1e-9, atol=1e-12)
                assert np.allclose(l[b, i], rl.numpy(), rtol=1e-12, atol=1e-12)


def check_order_and_padding(run):
    inp, idx, cnt = sparse_case([300, 129], 2, 8, 64, seed=9)
    o, l = run(inp, idx, cnt)
    rng = np.random.default_rng(3)
    perm = idx.copy()
    for b in range(2):
        for i in range(2):
            n = cnt[b * 2 + i]
            perm[b, i, :n] = rng.permutation(perm[b, i, :n])
    o2, l2 = run(inp, perm, cnt)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14) and np.allclose(l, l2, rtol=1e-12, atol=1e-14)
    pad = np.full((2, 2, 64 + 20), -1, dtype=np.int32)
    cnt_pad = cnt.copy()
    for b in range(2):
        for i in range(2):
            n = cnt[b * 2 + i]
            pos = np.sort(rng.choice(n + 20, size=n, replace=False))
            pad[b, i, pos] = idx[b, i, :n]
            cnt_pad[b * 2 + i] = n + 20
    o3, l3 = run(inp, pad, cnt_pad)
    assert np.array_equal(o, o3) and np.array_equal(l, l3)


def check_counts(run):
    inp, idx, cnt = sparse_case([200, 90], 1, 4, 40, seed=4)
    garbage = idx.copy()
    for b in range(2):
        n = cnt[b]
        garbage[b, 0, n:] = np.arange(40 - n) % 7          # valid tokens that must not be read
    o, l = run(inp, idx, cnt)
    o2, l2 = run(inp, garbage, cnt)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def check_single_and_empty(run):
    inp, _, _ = sparse_case([150], 1, 4, 4, seed=2)
    idx = np.array([[[77, -1, -1, -1]]], dtype=np.int32)
    o, l = run(inp, idx, np.array([4], np.int32))
    v = gather_rows(inp, 0, [77])[0]
    assert np.array_equal(o[0, 0], np.broadcast_to(v[:512], (4, 512)))
    Q = wl.bf16_bits_to_f32(inp.q[0, 0]).astype(np.float64)
    assert np.allclose(l[0, 0], inp.softmax_scale * (Q @ v), rtol=1e-13, atol=1e-13)
    o, l = run(inp, np.full((1, 1, 4), -1, np.int32), np.array([4], np.int32))
    assert (o == 0).all() and np.isneginf(l).all()
    o, l = run(inp, np.array([[[5, 6, 7, 8]]], np.int32), np.array([0], np.int32))
    assert (o == 0).all() and np.isneginf(l).all()


CHECKS = [check_dense, check_library, check_order_and_padding, check_counts, check_single_and_empty]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_sparse_oracle_pin(check):
    check(_run(oracle.load()))


MUTANTS = {
    "padding_ends_the_list": ("if (t < 0) continue;", "if (t < 0) break;"),
    "counts_ignored": ("const int n = a->counts[(long)b * a->s_q + i];", "const int n = a->topk;"),
    "list_of_first_token": ("const int32_t* list = a->indices + ((long)b * a->s_q + i) * a->topk;",
                            "const int32_t* list = a->indices + ((long)b * a->s_q) * a->topk;"),
    "table_of_first_sequence": ("const long blk = a->block_table[(long)b * a->max_blocks + t / a->page];",
                                "const long blk = a->block_table[t / a->page];"),
    "row_in_block": ("rows[used++] = a->kcache + (blk * a->page + t % a->page) * (long)a->d_qk;",
                     "rows[used++] = a->kcache + (blk * a->page + t / a->page) * (long)a->d_qk;"),
    "scale_dropped": ("score[u] = a->scale * dot;", "score[u] = dot;"),
    "rope_dropped": ("for (int d = 0; d < a->d_qk; ++d) dot +=", "for (int d = 0; d < a->d_v; ++d) dot +="),
    "lse_without_max": ("a->lse[row] = m + log(z);", "a->lse[row] = log(z);"),
    "not_normalised": ("const double w = exp(score[u] - m) / z;", "const double w = exp(score[u] - m);"),
    "last_listed_dropped": ("for (int u = 0; u < used; ++u) {\n        const double w",
                            "for (int u = 0; u + 1 < used; ++u) {\n        const double w"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = oracle._SRC_SPARSE.read_text()
    assert src.count(old) == 1, "mutation anchor not found: " + name
    tmp = Path(tempfile.mkdtemp(prefix="sparse_mutant_"))
    try:
        msrc = tmp / "mutant.c"
        msrc.write_text(src.replace(old, new))
        lib = oracle.load(oracle.build(force=True, src=[oracle._SRC, msrc], out=tmp / "libmutant.so"))
        failed = []
        for check in CHECKS:
            try:
                with np.errstate(all="ignore"):
                    check(_run(lib))
            except (AssertionError, RuntimeError, ValueError, IndexError):
                failed.append(check.__name__)
        assert failed, "planted mistake %s passed every pin" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
