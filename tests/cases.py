"""Test-side helpers: golden closed-form cases and small seeded decode batches.

Holds no attention arithmetic of its own (expected values come from the
fixtures' hand derivations, from library routines, or from the oracle).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_form_cases.json")

_SCALES = {
    "ln(3)/2": math.log(3.0) / 2.0,
    "ln(192)/8": math.log(192.0) / 8.0,
    "1/sqrt(192)": 1.0 / math.sqrt(192.0),
}


def _val(x):
    if isinstance(x, str):
        return float(x)
    return float(x)


def golden_cases():
    with open(GOLDEN) as f:
        doc = json.load(f)
    out = []
    for c in doc["cases"]:
        B = len(c["cache_seqlens"])
        page, d_qk, d_v = c["page"], c["d_qk"], c["d_v"]
        q = np.zeros((B, c["s_q"], c["h_q"], d_qk), dtype=np.float32)
        for b, i, h, d, v in c["q"]:
            q[b, i, h, d] = v
        kc = np.zeros((c["nblocks"], page, d_qk), dtype=np.float32)
        for blk, r, d, v in c["kcache"]:
            kc[blk, r, d] = v
        kbits = wl.f32_to_bf16_bits(kc)
        table = np.array(c["block_table"], dtype=np.int32)
        lens = np.array(c["cache_seqlens"], dtype=np.int32)
        if c.get("poison_unread"):
            used = np.zeros(c["nblocks"], dtype=bool)
            for b in range(B):
                n = (int(lens[b]) + page - 1) // page
                for j in range(n):
                    used[table[b, j]] = True
                if n:
                    tail = int(lens[b]) - (n - 1) * page
                    kbits[table[b, n - 1], tail:, :] = wl.BF16_NAN
            kbits[~used] = wl.BF16_NAN
        exp_out = np.zeros((B, c["s_q"], c["h_q"], d_v), dtype=np.float64)
        for b, i, h, d, v in c["expected_out"]:
            exp_out[b, i, h, d] = v
        exp_lse = np.full((B, c["s_q"], c["h_q"]), np.nan)
        for b, i, h, v in c["expected_lse"]:
            exp_lse[b, i, h] = _val(v)
        inp = wl.DecodeInputs(name=c["name"], q=wl.f32_to_bf16_bits(q), kcache=kbits,
                              block_table=table, cache_seqlens=lens, s_q=c["s_q"], h_q=c["h_q"],
                              softmax_scale=_SCALES[c["softmax_scale_expr"]], causal=c["causal"])
        out.append((inp, exp_out, exp_lse))
    return out


def small_batch(seqlens, s_q=1, h_q=16, seed=123, causal=True, poison=True, scale=None):
    rng = np.random.default_rng(seed)
    kw = {} if scale is None else {"softmax_scale": scale}
    return wl.build_inputs(seqlens, s_q, h_q, rng, name="small", causal=causal, poison=poison, **kw)


def gather_dense_k(inp, b):
    """Sequence b's cached rows in token order (float64), by indexing the block table."""
    L = int(inp.cache_seqlens[b])
    n = (L + wl.PAGE - 1) // wl.PAGE
    if n == 0:
        return np.zeros((0, inp.kcache.shape[2]))
    rows = inp.kcache[inp.block_table[b, :n]].reshape(-1, inp.kcache.shape[2])[:L]
    return wl.bf16_bits_to_f32(rows).astype(np.float64)
