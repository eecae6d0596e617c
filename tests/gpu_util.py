"""GPU-side helpers for the parity tests: move seeded inputs to the device, run the
library through its C ABI, and compare with the oracle to the stated bar."""
from __future__ import annotations

import numpy as np
import torch

import mla_paged_latent_amd as mla

OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


def to_device(inp, device="cuda:0"):
    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return {
        "q": bf16(inp.q),
        "kcache": bf16(inp.kcache),
        "block_table": torch.from_numpy(inp.block_table).to(device),
        "cache_seqlens": torch.from_numpy(inp.cache_seqlens).to(device),
    }


def run_library(inp, dev=None, num_units=None, device="cuda:0"):
    """Plan + decode on the GPU. Returns (out float32 numpy, lse numpy, plan)."""
    dev = dev or to_device(inp, device)
    meta, splits = mla.mla_get_metadata(dev["cache_seqlens"], inp.h_q, inp.s_q, num_units=num_units)
    out, lse = mla.mla_decode_fwd(dev["q"], dev["kcache"], dev["block_table"], dev["cache_seqlens"],
                                  inp.softmax_scale, meta, splits, causal=inp.causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), (meta.cpu().numpy(), splits.cpu().numpy())


def assert_parity(out, lse, ref_out, ref_lse, what=""):
    """|out-ref| <= 1e-2 + 1e-2|ref| and |lse-ref| <= 1e-3; -inf lse must match exactly."""
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape, what
    assert np.isfinite(out).all(), what + ": non-finite out"
    err = np.abs(out - ref_out)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref_out)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError("%s: out mismatch at %s: got %r ref %r (%d bad of %d)"
                             % (what, tuple(idx), float(out[tuple(idx)]), float(ref_out[tuple(idx)]),
                                int(bad.sum()), bad.size))
    inf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), inf_ref), what + ": -inf lse pattern differs"
    fin = ~inf_ref
    lerr = np.abs(lse[fin] - ref_lse[fin])
    if lerr.size and lerr.max() > LSE_ATOL:
        raise AssertionError("%s: lse mismatch, max err %.3g" % (what, float(lerr.max())))


def rel_rms(out, ref):
    return float(np.sqrt(np.mean((out - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
