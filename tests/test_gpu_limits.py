"""GPU parity at the limits the library accepts: s_q*h_q = 1024 (the most query
rows; 16 head groups of the 64-row kernel) and 1008 (63 head groups of the
16-row kernel), the largest batch (16,384 sequences; checked on sampled
sequences the oracle computes one by one) on both kernel shapes, and one
sequence of 131,072 cached tokens split over many units."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_paged_latent_amd as mla
import oracle
import workloads as wl
from tests import cases
from tests.gpu_util import assert_parity, run_library

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


@pytest.mark.parametrize("lens,s_q,h_q", [([300, 77], 8, 128), ([129, 5], 1, 1024), ([200, 3, 64], 1, 1008),
                                          ([90, 1], 7, 144)])
def test_most_query_rows(lens, s_q, h_q):
    _say("rows lens=%s s_q=%d h_q=%d" % (lens, s_q, h_q))
    inp = cases.small_batch(lens, s_q=s_q, h_q=h_q, seed=s_q * h_q + len(lens))
    out, lse, _ = run_library(inp)
    ro, rl = oracle.decode_inputs(inp)
    assert_parity(out, lse, ro, rl, "rows %d" % (s_q * h_q))


@pytest.mark.parametrize("h_q", [16, 64])
def test_largest_batch(h_q):
    """16,384 sequences of 1-96 tokens; sampled sequences against the oracle."""
    _say("largest batch h_q=%d" % h_q)
    rng = np.random.default_rng(h_q)
    lens = rng.integers(1, 97, 16384).astype(np.int32)
    lens[:3] = [0, 1, 64]
    inp = wl.build_inputs(lens, 1, h_q, rng, name="largest_batch", causal=True, poison=False)
    out, lse, _ = run_library(inp)
    pick = sorted({0, 1, 2, 16383, int(np.argmax(lens))} | set(rng.choice(16384, size=12, replace=False).tolist()))
    sub = wl.subset(inp, pick)
    ro, rl = oracle.decode_inputs(sub)
    assert_parity(out[pick], lse[pick], ro, rl, "largest batch")


@pytest.mark.parametrize("h_q", [16, 64])
def test_longest_sequence(h_q):
    """One sequence of 131,072 tokens next to a short one."""
    _say("longest sequence h_q=%d" % h_q)
    inp = cases.small_batch([131072, 70], s_q=1, h_q=h_q, seed=77 + h_q, poison=False)
    out, lse, _ = run_library(inp)
    ro, rl = oracle.decode_inputs(inp)
    assert_parity(out, lse, ro, rl, "longest sequence")
