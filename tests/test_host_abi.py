"""Host-side tests of the C ABI (no GPU): symbols, argument checks, the host planner.

The library is loaded but no device work is requested: every call here either
fails its host-side checks before any HIP call or runs purely on the host.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import mla_paged_latent_amd as mla

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "mla_paged_latent.h"

MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL = -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    if not mla.LIB_PATH.exists():
        from mla_paged_latent_amd import build
        build.build()
    return mla.load_library()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_two_calls():
    fns = declared_functions()
    assert "mla_get_metadata" in fns and "mla_decode_fwd" in fns, fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_no_torch_types_in_the_abi():
    text = HEADER.read_text()
    assert "torch" not in re.sub(r"/\*.*?\*/", "", text, flags=re.S).lower()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 99):
        assert lib.mla_status_string(code)


def _decode_args(**over):
    fake = ctypes.c_void_p(0x10000)      # never dereferenced: the checks fail first
    a = dict(q=fake, kcache=fake, nblocks=8, block_table=fake, max_blocks=4, cache_seqlens=fake, batch=2,
             s_q=1, h_q=16, scale=0.07, causal=1, meta=fake, splits=fake, units=8, out=fake, lse=fake,
             ws=fake, ws_bytes=1 << 40, stream=None)
    a.update(over)
    return [a[k] for k in ("q", "kcache", "nblocks", "block_table", "max_blocks", "cache_seqlens", "batch",
                           "s_q", "h_q", "scale", "causal", "meta", "splits", "units", "out", "lse", "ws",
                           "ws_bytes", "stream")]


@pytest.mark.parametrize("over,code", [
    (dict(q=None), MLA_ERR_INVALID_ARG),
    (dict(kcache=None), MLA_ERR_INVALID_ARG),
    (dict(out=None), MLA_ERR_INVALID_ARG),
    (dict(ws=None), MLA_ERR_INVALID_ARG),
    (dict(batch=0), MLA_ERR_INVALID_ARG),
    (dict(nblocks=0), MLA_ERR_INVALID_ARG),
    (dict(max_blocks=0), MLA_ERR_INVALID_ARG),
    (dict(units=0), MLA_ERR_INVALID_ARG),
    (dict(units=2), MLA_ERR_INVALID_ARG),                        # per-sequence plan needs batch + 1
    (dict(scale=float("nan")), MLA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), MLA_ERR_INVALID_ARG),
    (dict(q=ctypes.c_void_p(0x10008)), MLA_ERR_INVALID_ARG),      # misaligned
    (dict(h_q=15), MLA_ERR_UNSUPPORTED),
    (dict(s_q=3, h_q=8), MLA_ERR_UNSUPPORTED),                    # 24 rows
    (dict(s_q=16, h_q=128), MLA_ERR_UNSUPPORTED),                 # 2048 rows
    (dict(batch=16385), MLA_ERR_UNSUPPORTED),
    (dict(ws_bytes=1024), MLA_ERR_WORKSPACE_TOO_SMALL),
])
@pytest.mark.parametrize("name", ["mla_decode_fwd", "mla_decode_fwd_splits", "mla_decode_fp8_fwd",
                                  "mla_decode_fp8_fwd_splits"])
def test_decode_rejects_bad_arguments_before_any_launch(lib, name, over, code):
    args = _decode_args(**over)
    if "fp8" in name:
        args.insert(2, ctypes.c_void_p(0x20000))          # kscale
    assert getattr(lib, name)(*args) == code


@pytest.mark.parametrize("name", ["mla_decode_sparse_fwd", "mla_decode_sparse_fwd_splits"])
@pytest.mark.parametrize("over,code", [
    (dict(q=None), MLA_ERR_INVALID_ARG),
    (dict(indices=None), MLA_ERR_INVALID_ARG),
    (dict(units=2), MLA_ERR_INVALID_ARG),                        # needs batch * s_q + 1
    (dict(topk=2049), MLA_ERR_UNSUPPORTED),
    (dict(h_q=24), MLA_ERR_UNSUPPORTED),
    (dict(ws_bytes=1024), MLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_sparse_decode_rejects_bad_arguments_before_any_launch(lib, name, over, code):
    fake = ctypes.c_void_p(0x10000)
    a = dict(q=fake, kcache=fake, nblocks=8, block_table=fake, max_blocks=4, indices=fake, lens=fake, topk=64,
             batch=2, s_q=1, h_q=16, scale=0.07, meta=fake, splits=fake, units=8, out=fake, lse=fake, ws=fake,
             ws_bytes=1 << 40, stream=None)
    a.update(over)
    args = [a[k] for k in ("q", "kcache", "nblocks", "block_table", "max_blocks", "indices", "lens", "topk", "batch",
                           "s_q", "h_q", "scale", "meta", "splits", "units", "out", "lse", "ws", "ws_bytes", "stream")]
    assert getattr(lib, name)(*args) == code


def test_get_metadata_rejects_bad_arguments(lib):
    fake = ctypes.c_void_p(0x10000)
    assert lib.mla_get_metadata(None, 2, 1, 16, 8, fake, fake, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_get_metadata(fake, 2, 1, 16, 0, fake, fake, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_get_metadata(fake, 2, 1, 17, 8, fake, fake, None) == MLA_ERR_UNSUPPORTED


def test_plan_sizes(lib):
    # 16 query rows per workgroup: 7/8 of the CUs
    s = mla.mla_plan_sizes(16, 1, 16, num_cus=256)
    assert s["num_units"] == 224
    assert s["meta_bytes"] == 224 * 8 * 4 and s["splits_bytes"] == 17 * 4
    assert s["workspace_bytes"] == mla.mla_workspace_bytes(16, 1, 16, 224)
    assert mla.mla_plan_sizes(300, 1, 16, num_cus=256)["num_units"] == 301
    # 64 query rows per workgroup: h_q=128, s_q=2 is 256 rows = four head groups
    assert mla.mla_plan_sizes(128, 2, 128, num_cus=256)["num_units"] == 64
    assert mla.mla_plan_sizes(64, 1, 128, num_cus=256)["num_units"] == 128
    # 192 rows = three head groups
    assert mla.mla_plan_sizes(64, 3, 64, num_cus=256)["num_units"] == 85
    assert mla.mla_plan_sizes(64, 1, 64, num_cus=256)["num_units"] == 256
    # 48 rows: three head groups of 16, per-sequence plan (224 CUs' worth)
    assert mla.mla_plan_sizes(8, 3, 16, num_cus=256)["num_units"] == 74
    with pytest.raises(mla.MLAError):
        mla.mla_plan_sizes(4, 1, 10, num_cus=256)


# ------------------------------------------------------------- planner properties

def blocks(L):
    return (np.asarray(L, dtype=np.int64) + 63) // 64


def kind_and_width(lens, s_q, h_q, units):
    """Plan shape the library uses and its block budget per unit."""
    rows = s_q * h_q
    nb = blocks(lens)
    if rows % 64 == 0:
        kappa = 4
        total = int(nb.sum()) + kappa * int((nb > 0).sum())
        return "cost_line", kappa, max(1, -(-total // units))
    return "by_sequence", 0, max(1, -(-int(nb.sum()) // (units - len(lens))))


def check_plan(lens, s_q, h_q, units, meta, splits):
    """Every block owned by exactly one unit, units contiguous, split counts and indices consistent,
    balance bound of the plan shape."""
    lens = np.asarray(lens)
    B = len(lens)
    nb = blocks(lens)
    kind, kappa, W = kind_and_width(lens, s_q, h_q, units)
    owner = {}
    touched = [set() for _ in range(B)]
    for u in range(units):
        b0, j0, b1, j1, split = (int(x) for x in meta[u, :5])
        assert (b0, j0) <= (b1, j1)
        if kind == "by_sequence" and b0 < B:
            assert b0 == b1, "a per-sequence unit spans sequences"
        cost = 0
        first = True
        b, j = b0, j0
        while (b, j) < (b1, j1) and b < B:
            if j >= nb[b]:
                b, j = b + 1, 0
                continue
            assert (b, j) not in owner
            owner[(b, j)] = u
            if u not in touched[b]:
                touched[b].add(u)
                cost += kappa
                if first:
                    # the split index of the first segment counts earlier units on b
                    assert split == len([x for x in touched[b] if x < u])
                first = False
            cost += 1
            j += 1
        assert cost <= W + kappa, (u, cost, W)
    for b in range(B):
        for j in range(int(nb[b])):
            assert (b, j) in owner, (b, j)
        us = [owner[(b, j)] for j in range(int(nb[b]))]
        assert us == sorted(us)
    ns = np.array([len(t) for t in touched])
    assert splits[0] == 0 and np.array_equal(np.diff(splits), ns)
    assert splits[-1] <= units + B
    # trailing fields: length, partial slot and split count of the first sequence
    for u in range(units):
        b0, j0, b1, j1, split, L, slot, nsplit = (int(x) for x in meta[u])
        if b0 < B and (b0, j0) != (b1, j1):
            assert L == lens[b0] and slot == splits[b0] + split and nsplit == ns[b0]
        else:
            assert (L, slot, nsplit) == (0, 0, 0)


@pytest.mark.parametrize("seed", range(12))
def test_host_plan_properties(lib, seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 300))
    lens = rng.integers(0, 5000, B)
    lens[rng.random(B) < 0.1] = 0
    s_q, h_q = [(1, 16), (2, 16), (1, 128), (2, 128), (3, 16), (1, 32), (2, 32), (1, 64)][seed % 8]
    units = int(rng.choice([1, 3, 64, 128, 256, 1000]))
    if (s_q * h_q) % 64 != 0:
        units += B
    meta, splits = mla.mla_get_metadata_host(lens, h_q, s_q, units)
    check_plan(lens, s_q, h_q, units, meta, splits)


def test_host_plan_workloads(lib):
    import workloads as wl
    for name in wl.WORKLOADS:
        rng = np.random.default_rng(wl.WORKLOADS[name])
        lens = wl._seqlens(name, rng)
        s_q, h_q, _ = wl._shape(name)
        units = mla.mla_plan_sizes(len(lens), s_q, h_q, num_cus=256)["num_units"]
        meta, splits = mla.mla_get_metadata_host(lens, h_q, s_q, units)
        check_plan(lens, s_q, h_q, units, meta, splits)


def test_host_plan_all_empty(lib):
    for h_q in (16, 128):
        meta, splits = mla.mla_get_metadata_host([0, 0, 0], h_q, 1, 8)
        assert np.array_equal(splits, [0, 0, 0, 0])
        assert (meta[:, 0] == 3).all()          # every unit starts past the batch


def test_per_sequence_plan_needs_a_unit_per_sequence(lib):
    with pytest.raises(mla.MLAError):
        mla.mla_get_metadata_host([10, 20, 30], 16, 1, 3)
    meta, splits = mla.mla_get_metadata_host([10, 20, 30], 16, 1, 4)
    assert splits[-1] == 3


def test_noalloc_decode_refuses_more_than_its_scratch_before_any_hip_call(lib):
    """The allocation-free decode checks its arguments and the workspace the call needs
    against the fixed scratch (MLA_NOALLOC_SCRATCH_BYTES = 128 MiB) before it touches the
    GPU: the mixed workload's plan fits, a larger batch or more units does not."""
    args = _decode_args()
    ok_units = mla.mla_plan_sizes(128, 2, 128, num_cus=256)["num_units"]
    assert mla.mla_workspace_bytes(128, 2, 128, ok_units) <= 128 << 20
    assert mla.mla_workspace_bytes(256, 2, 128, 256) > 128 << 20

    def call(**over):
        a = _decode_args(**over)
        return lib.mla_decode_fwd_noalloc(*(a[:16] + [a[18]]))
    assert call(batch=256, s_q=2, h_q=128, units=256, max_blocks=300) == MLA_ERR_WORKSPACE_TOO_SMALL
    assert call(batch=16, s_q=1, h_q=16, units=100000) == MLA_ERR_WORKSPACE_TOO_SMALL
    assert call(q=None) == MLA_ERR_INVALID_ARG
    assert call(h_q=15) == MLA_ERR_UNSUPPORTED
    assert call(units=2) == MLA_ERR_INVALID_ARG


def test_check_inputs_host_accepts_the_workloads_and_names_the_first_bad_sequence(lib):
    import workloads as wl
    for name in wl.WORKLOADS:
        inp = wl.make_workload(name, poison=False)
        assert mla.mla_check_inputs_host(inp.cache_seqlens, inp.block_table, inp.kcache.shape[0]) == -1, name
    inp = wl.make_workload("memory_bound", poison=False)
    nb = inp.kcache.shape[0]
    lens, table = inp.cache_seqlens.copy(), inp.block_table.copy()
    used = (lens + 63) // 64
    # entries past each sequence's last block are never read: -1 there is fine (the recipe pads with -1)
    assert (table[0, used[0]:] == -1).all() or used[0] == table.shape[1]
    for b, bad in ((3, -1), (5, nb), (9, 1 << 30)):
        t = table.copy()
        t[b, used[b] - 1] = bad
        assert mla.mla_check_inputs_host(lens, t, nb) == b
    l2 = lens.copy()
    l2[7] = 64 * table.shape[1] + 1                     # longer than the table can hold
    assert mla.mla_check_inputs_host(l2, table, nb) == 7
    l2 = lens.copy()
    l2[2] = -5
    assert mla.mla_check_inputs_host(l2, table, nb) == 2
    assert mla.mla_check_inputs_host(lens, table, int(table.max())) == int(np.argmax((table == table.max()).any(1)))
