"""MLA decode over a paged latent KV cache on MI355X (gfx950).

Thin ctypes binding of the C ABI in include/mla_paged_latent.h. Each Python
function has the name of the C entry point it calls and only marshals
arguments: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and the current stream. The library must be
built first (python -m mla_paged_latent_amd.build); nothing here falls back to
another implementation.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from pathlib import Path

import numpy as np

LIB_PATH = Path(__file__).resolve().parent / "libmla_paged_latent.so"

D_QK = 576
D_V = 512
PAGE_SIZE = 64
META_INTS = 8

MLA_OK = 0

_lib = None


class MLAError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (func, status_string(status), status))


def load_library(path: Path | str | None = None):
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    # MLA_LIB names another build of the same sources (the tests' sanitizer build of the host code)
    p = Path(path) if path is not None else Path(os.environ.get("MLA_LIB") or LIB_PATH)
    if not p.exists():
        raise RuntimeError("HIP library %s is not built; run `python -m mla_paged_latent_amd.build`" % p)
    lib = ctypes.CDLL(str(p))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [i32]
    lib.mla_plan_sizes.restype = i32
    lib.mla_plan_sizes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(sz),
                                   ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_workspace_bytes.restype = i32
    lib.mla_workspace_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.mla_get_metadata.restype = i32
    lib.mla_get_metadata.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.mla_get_metadata_host.restype = i32
    lib.mla_get_metadata_host.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    dec = [vp, vp, i64, vp, i32, vp, i32, i32, i32, ctypes.c_float, i32, vp, vp, i32, vp, vp, vp, sz, vp]
    for name in ("mla_decode_fwd", "mla_decode_fwd_splits"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = dec
    lib.mla_decode_fwd_noalloc.restype = i32
    lib.mla_decode_fwd_noalloc.argtypes = dec[:16] + [vp]
    lib.mla_check_inputs_host.restype = i32
    lib.mla_check_inputs_host.argtypes = [vp, i32, vp, i32, i64, ctypes.POINTER(i32)]
    lib.mla_combine_splits.restype = i32
    lib.mla_combine_splits.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.mla_sparse_plan_sizes.restype = i32
    lib.mla_sparse_plan_sizes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(sz),
                                          ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_get_metadata_sparse.restype = i32
    lib.mla_get_metadata_sparse.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    for name in ("mla_decode_sparse_fwd", "mla_decode_sparse_fwd_splits"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [vp, vp, i64, vp, i32, vp, vp, i32, i32, i32, i32, ctypes.c_float,
                                       vp, vp, i32, vp, vp, vp, sz, vp]
    lib.mla_fp8_plan_sizes.restype = i32
    lib.mla_fp8_plan_sizes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(sz),
                                       ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_get_metadata_fp8.restype = i32
    lib.mla_get_metadata_fp8.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    for name in ("mla_decode_fp8_fwd", "mla_decode_fp8_fwd_splits"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, i32, i32, ctypes.c_float, i32, vp, vp,
                                       i32, vp, vp, vp, sz, vp]
    lib.mla_append_kv_fp8.restype = i32
    lib.mla_append_kv_fp8.argtypes = [vp, vp, i64, vp, i32, vp, vp, i32, i32, vp]
    lib.mla_append_kv.restype = i32
    lib.mla_append_kv.argtypes = [vp, i64, vp, i32, vp, vp, i32, i32, vp]
    lib.mla_block_pool_create.restype = i32
    lib.mla_block_pool_create.argtypes = [i64, i32, i32, ctypes.POINTER(vp)]
    lib.mla_block_pool_destroy.restype = None
    lib.mla_block_pool_destroy.argtypes = [vp]
    lib.mla_block_pool_reserve.restype = i32
    lib.mla_block_pool_reserve.argtypes = [vp, i32, i32]
    lib.mla_block_pool_release.restype = i32
    lib.mla_block_pool_release.argtypes = [vp, i32]
    lib.mla_block_pool_free_blocks.restype = i64
    lib.mla_block_pool_free_blocks.argtypes = [vp]
    lib.mla_block_pool_table.restype = i32
    lib.mla_block_pool_table.argtypes = [vp, vp, i32, i32, vp, vp]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mla_status_string(int(status)).decode()


def _check(func: str, rc: int):
    if rc != MLA_OK:
        raise MLAError(func, rc)


def mla_plan_sizes(batch: int, s_q: int, h_q: int, num_cus: int = 0) -> dict:
    """Plan geometry and buffer sizes (host only). num_cus <= 0 asks the current device."""
    lib = load_library()
    units = ctypes.c_int(0)
    meta, splits, ws = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_plan_sizes", lib.mla_plan_sizes(batch, s_q, h_q, num_cus, ctypes.byref(units),
                                                ctypes.byref(meta), ctypes.byref(splits), ctypes.byref(ws)))
    return {"num_units": units.value, "meta_bytes": meta.value, "splits_bytes": splits.value,
            "workspace_bytes": ws.value}


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on(torch, dev):
    """Make dev the current device for the call (no-op when it already is)."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _need(t, dtype, name, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def mla_workspace_bytes(batch: int, s_q: int, h_q: int, num_units: int) -> int:
    return workspace_bytes(batch, s_q, h_q, num_units)


def mla_get_metadata(cache_seqlens, h_q: int, s_q: int = 1, num_units: int | None = None, tile_meta=None,
                     num_splits=None):
    """Split-KV tile plan on the device. Returns (tile_meta int32 [G, 8], num_splits int32 [B+1]);
    pass tile_meta / num_splits to fill existing buffers."""
    import torch
    _need(cache_seqlens, torch.int32, "cache_seqlens")
    B = int(cache_seqlens.shape[0])
    dev = cache_seqlens.device
    with _on(torch, dev):
        if num_units is None:
            num_units = mla_plan_sizes(B, s_q, h_q)["num_units"]
        if tile_meta is None:
            tile_meta = torch.empty((num_units, META_INTS), dtype=torch.int32, device=dev)
        if num_splits is None:
            num_splits = torch.empty((B + 1,), dtype=torch.int32, device=dev)
        _need(tile_meta, torch.int32, "tile_meta", dev)
        _need(num_splits, torch.int32, "num_splits", dev)
        if tuple(tile_meta.shape) != (num_units, META_INTS) or tuple(num_splits.shape) != (B + 1,):
            raise ValueError("tile_meta must be [num_units, 8] and num_splits [B + 1]")
        _check("mla_get_metadata", load_library().mla_get_metadata(
            cache_seqlens.data_ptr(), B, s_q, h_q, num_units, tile_meta.data_ptr(), num_splits.data_ptr(),
            _stream(torch)))
    return tile_meta, num_splits


def mla_get_metadata_host(cache_seqlens, h_q: int, s_q: int, num_units: int):
    """The same plan computed by the library on the host (numpy in, numpy out)."""
    lens = np.ascontiguousarray(np.asarray(cache_seqlens), dtype=np.int32)
    B = int(lens.shape[0])
    meta = np.zeros((num_units, META_INTS), dtype=np.int32)
    splits = np.zeros((B + 1,), dtype=np.int32)
    _check("mla_get_metadata_host", load_library().mla_get_metadata_host(
        lens.ctypes.data, B, s_q, h_q, num_units, meta.ctypes.data, splits.ctypes.data))
    return meta, splits


def _decode_args(q, kcache, block_table, cache_seqlens, softmax_scale, tile_meta, num_splits, causal, out, lse,
                 workspace):
    import torch
    _need(q, torch.bfloat16, "q")
    dev = q.device
    _need(kcache, torch.bfloat16, "kcache", dev)
    _need(block_table, torch.int32, "block_table", dev)
    _need(cache_seqlens, torch.int32, "cache_seqlens", dev)
    _need(tile_meta, torch.int32, "tile_meta", dev)
    _need(num_splits, torch.int32, "num_splits", dev)
    if q.dim() != 4 or q.shape[3] != D_QK:
        raise ValueError("q must be [B, s_q, h_q, 576]")
    if kcache.dim() != 3 or kcache.shape[1] != PAGE_SIZE or kcache.shape[2] != D_QK:
        raise ValueError("kcache must be [nblocks, 64, 576]")
    B, s_q, h_q, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and cache_seqlens [B]")
    if tile_meta.dim() != 2 or tile_meta.shape[1] != META_INTS or tuple(num_splits.shape) != (B + 1,):
        raise ValueError("tile_meta / num_splits do not look like a plan for this batch")
    num_units = int(tile_meta.shape[0])
    if out is None:
        out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    _need(out, torch.bfloat16, "out", dev)
    _need(lse, torch.float32, "lse", dev)
    if tuple(out.shape) != (B, s_q, h_q, D_V) or tuple(lse.shape) != (B, s_q, h_q):
        raise ValueError("out / lse have the wrong shape")
    if workspace is None:
        ws_bytes = workspace_bytes(B, s_q, h_q, num_units)
        workspace = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", dev)
    args = (q.data_ptr(), kcache.data_ptr(), int(kcache.shape[0]), block_table.data_ptr(), int(block_table.shape[1]),
            cache_seqlens.data_ptr(), B, s_q, h_q, float(softmax_scale), 1 if causal else 0, tile_meta.data_ptr(),
            num_splits.data_ptr(), num_units, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
            int(workspace.numel()), _stream(torch))
    return args, out, lse, workspace


def mla_decode_fwd(q, kcache, block_table, cache_seqlens, softmax_scale: float, tile_meta, num_splits,
                   causal: bool = True, out=None, lse=None, workspace=None):
    """Decode attention. q bf16 [B, s_q, h_q, 576], kcache bf16 [nblocks, 64, 576],
    block_table int32 [B, max_blocks], cache_seqlens int32 [B].
    Returns (out bf16 [B, s_q, h_q, 512], lse float32 [B, s_q, h_q])."""
    import torch
    with _on(torch, q.device):
        args, out, lse, _ = _decode_args(q, kcache, block_table, cache_seqlens, softmax_scale, tile_meta,
                                         num_splits, causal, out, lse, workspace)
        _check("mla_decode_fwd", load_library().mla_decode_fwd(*args))
    return out, lse


def mla_decode_fwd_splits(q, kcache, block_table, cache_seqlens, softmax_scale: float, tile_meta, num_splits,
                          causal: bool = True, out=None, lse=None, workspace=None):
    """First stage of mla_decode_fwd only (the decode kernel): unsplit sequences get
    out/lse, split ones leave partials in workspace. Returns (out, lse, workspace)."""
    import torch
    with _on(torch, q.device):
        args, out, lse, workspace = _decode_args(q, kcache, block_table, cache_seqlens, softmax_scale, tile_meta,
                                                 num_splits, causal, out, lse, workspace)
        _check("mla_decode_fwd_splits", load_library().mla_decode_fwd_splits(*args))
    return out, lse, workspace


def mla_decode_fwd_noalloc(q, kcache, block_table, cache_seqlens, softmax_scale: float, tile_meta, num_splits,
                           causal: bool = True, out=None, lse=None):
    """mla_decode_fwd with the split partials in the library's fixed device scratch
    (no workspace; the C call allocates nothing). out / lse are allocated here when
    not given. Returns (out, lse)."""
    import torch
    with _on(torch, q.device):
        dummy = torch.empty((16,), dtype=torch.uint8, device=q.device)
        args, out, lse, _ = _decode_args(q, kcache, block_table, cache_seqlens, softmax_scale, tile_meta,
                                         num_splits, causal, out, lse, dummy)
        _check("mla_decode_fwd_noalloc", load_library().mla_decode_fwd_noalloc(*(args[:16] + (args[18],))))
    return out, lse


def mla_combine_splits(num_splits, s_q: int, h_q: int, num_units: int, out, lse, workspace):
    """Second stage of mla_decode_fwd only (the split combine kernel)."""
    import torch
    _need(num_splits, torch.int32, "num_splits")
    B = int(num_splits.shape[0]) - 1
    with _on(torch, num_splits.device):
        _check("mla_combine_splits", load_library().mla_combine_splits(
            num_splits.data_ptr(), B, s_q, h_q, num_units, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
            int(workspace.numel()), _stream(torch)))
    return out, lse


def mla_check_inputs_host(cache_seqlens, block_table, nblocks: int):
    """Check the decode calls' contract on host arrays (numpy): 0 <= L_b <= 64 * max_blocks and
    every used table entry in [0, nblocks). Returns -1 when it holds, else the first bad sequence."""
    lens = np.ascontiguousarray(np.asarray(cache_seqlens), dtype=np.int32)
    table = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    if table.ndim != 2 or table.shape[0] != lens.shape[0]:
        raise ValueError("block_table must be [B, max_blocks] and cache_seqlens [B]")
    bad = ctypes.c_int(-2)
    rc = load_library().mla_check_inputs_host(lens.ctypes.data, int(lens.shape[0]), table.ctypes.data,
                                              int(table.shape[1]), int(nblocks), ctypes.byref(bad))
    if rc != MLA_OK and bad.value < 0:
        raise MLAError("mla_check_inputs_host", rc)
    return bad.value


def mla_sparse_plan_sizes(batch: int, s_q: int, h_q: int, topk: int, num_cus: int = 0) -> dict:
    """Plan geometry and buffer sizes of a sparse decode batch (host only)."""
    units = ctypes.c_int(0)
    meta, splits, ws = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_sparse_plan_sizes", load_library().mla_sparse_plan_sizes(
        batch, s_q, h_q, topk, num_cus, ctypes.byref(units), ctypes.byref(meta), ctypes.byref(splits),
        ctypes.byref(ws)))
    return {"num_units": units.value, "meta_bytes": meta.value, "splits_bytes": splits.value,
            "workspace_bytes": ws.value}


def mla_get_metadata_sparse(topk_lens, batch: int, s_q: int, h_q: int, topk: int, num_units: int | None = None,
                            tile_meta=None, num_splits=None):
    """Split plan of a sparse batch on the device from topk_lens int32 [batch * s_q].
    Returns (tile_meta int32 [G, 8], num_splits int32 [batch * s_q + 1])."""
    import torch
    _need(topk_lens, torch.int32, "topk_lens")
    dev = topk_lens.device
    if tuple(topk_lens.shape) != (batch * s_q,):
        raise ValueError("topk_lens must be [batch * s_q]")
    with _on(torch, dev):
        if num_units is None:
            num_units = mla_sparse_plan_sizes(batch, s_q, h_q, topk)["num_units"]
        if tile_meta is None:
            tile_meta = torch.empty((num_units, META_INTS), dtype=torch.int32, device=dev)
        if num_splits is None:
            num_splits = torch.empty((batch * s_q + 1,), dtype=torch.int32, device=dev)
        _check("mla_get_metadata_sparse", load_library().mla_get_metadata_sparse(
            topk_lens.data_ptr(), batch, s_q, h_q, topk, num_units, tile_meta.data_ptr(), num_splits.data_ptr(),
            _stream(torch)))
    return tile_meta, num_splits


def mla_decode_sparse_fwd(q, kcache, block_table, indices, topk_lens, softmax_scale: float, tile_meta, num_splits,
                          out=None, lse=None, workspace=None):
    """Sparse decode: q bf16 [B, s_q, h_q, 576] attends, per new token, over the
    cached positions indices[b, i, :topk_lens[b*s_q+i]] (int32 [B, s_q, topk];
    entries < 0 are padding). Returns (out bf16 [B, s_q, h_q, 512], lse f32 [B, s_q, h_q])."""
    out, lse, _ = _sparse_call("mla_decode_sparse_fwd", q, kcache, block_table, indices, topk_lens, softmax_scale,
                               tile_meta, num_splits, out, lse, workspace)
    return out, lse


def mla_decode_sparse_fwd_splits(q, kcache, block_table, indices, topk_lens, softmax_scale: float, tile_meta,
                                 num_splits, out=None, lse=None, workspace=None):
    """The decode kernel of mla_decode_sparse_fwd alone: unsplit lists get out/lse, split
    ones leave partials in workspace (merged by mla_combine_splits with B * s_q lists of
    one new token). Returns (out, lse, workspace)."""
    return _sparse_call("mla_decode_sparse_fwd_splits", q, kcache, block_table, indices, topk_lens, softmax_scale,
                        tile_meta, num_splits, out, lse, workspace)


def _sparse_call(name, q, kcache, block_table, indices, topk_lens, softmax_scale, tile_meta, num_splits, out, lse,
                 workspace):
    import torch
    _need(q, torch.bfloat16, "q")
    dev = q.device
    _need(kcache, torch.bfloat16, "kcache", dev)
    _need(block_table, torch.int32, "block_table", dev)
    _need(indices, torch.int32, "indices", dev)
    _need(topk_lens, torch.int32, "topk_lens", dev)
    _need(tile_meta, torch.int32, "tile_meta", dev)
    _need(num_splits, torch.int32, "num_splits", dev)
    if q.dim() != 4 or q.shape[3] != D_QK:
        raise ValueError("q must be [B, s_q, h_q, 576]")
    if kcache.dim() != 3 or kcache.shape[1] != PAGE_SIZE or kcache.shape[2] != D_QK:
        raise ValueError("kcache must be [nblocks, 64, 576]")
    B, s_q, h_q, _ = q.shape
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, s_q) or tuple(topk_lens.shape) != (B * s_q,):
        raise ValueError("indices must be [B, s_q, topk] and topk_lens [B * s_q]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    topk = int(indices.shape[2])
    num_units = int(tile_meta.shape[0])
    with _on(torch, dev):
        if out is None:
            out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
        if workspace is None:
            ws = mla_sparse_plan_sizes(B, s_q, h_q, topk)["workspace_bytes"]
            n = ctypes.c_size_t(0)
            _check("mla_workspace_bytes", load_library().mla_workspace_bytes(B * s_q, 1, h_q, num_units,
                                                                              ctypes.byref(n)))
            workspace = torch.empty((max(ws, n.value, 16),), dtype=torch.uint8, device=dev)
        _check(name, getattr(load_library(), name)(
            q.data_ptr(), kcache.data_ptr(), int(kcache.shape[0]), block_table.data_ptr(), int(block_table.shape[1]),
            indices.data_ptr(), topk_lens.data_ptr(), topk, B, s_q, h_q, float(softmax_scale), tile_meta.data_ptr(),
            num_splits.data_ptr(), num_units, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
            int(workspace.numel()), _stream(torch)))
    return out, lse, workspace


def mla_fp8_plan_sizes(batch: int, s_q: int, h_q: int, num_cus: int = 0) -> dict:
    """Plan geometry and buffer sizes for the FP8-cache decode (host only)."""
    units = ctypes.c_int(0)
    meta, splits, ws = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_fp8_plan_sizes", load_library().mla_fp8_plan_sizes(batch, s_q, h_q, num_cus, ctypes.byref(units),
                                                                    ctypes.byref(meta), ctypes.byref(splits),
                                                                    ctypes.byref(ws)))
    return {"num_units": units.value, "meta_bytes": meta.value, "splits_bytes": splits.value,
            "workspace_bytes": ws.value}


def mla_get_metadata_fp8(cache_seqlens, h_q: int, s_q: int = 1, num_units: int | None = None, tile_meta=None,
                         num_splits=None):
    """Split plan for the FP8-cache decode (device). Returns (tile_meta, num_splits)."""
    import torch
    _need(cache_seqlens, torch.int32, "cache_seqlens")
    B = int(cache_seqlens.shape[0])
    dev = cache_seqlens.device
    with _on(torch, dev):
        if num_units is None:
            num_units = mla_fp8_plan_sizes(B, s_q, h_q)["num_units"]
        if tile_meta is None:
            tile_meta = torch.empty((num_units, META_INTS), dtype=torch.int32, device=dev)
        if num_splits is None:
            num_splits = torch.empty((B + 1,), dtype=torch.int32, device=dev)
        _check("mla_get_metadata_fp8", load_library().mla_get_metadata_fp8(
            cache_seqlens.data_ptr(), B, s_q, h_q, num_units, tile_meta.data_ptr(), num_splits.data_ptr(),
            _stream(torch)))
    return tile_meta, num_splits


def mla_decode_fp8_fwd(q, kcodes, kscale, block_table, cache_seqlens, softmax_scale: float, tile_meta, num_splits,
                       causal: bool = True, out=None, lse=None, workspace=None):
    """Decode over an FP8 cache: kcodes uint8 [nblocks, 64, 576] (E4M3), kscale float32
    [nblocks, 64]; the rest as mla_decode_fwd. Returns (out, lse)."""
    out, lse, _ = _fp8_call("mla_decode_fp8_fwd", q, kcodes, kscale, block_table, cache_seqlens, softmax_scale,
                            tile_meta, num_splits, causal, out, lse, workspace)
    return out, lse


def mla_decode_fp8_fwd_splits(q, kcodes, kscale, block_table, cache_seqlens, softmax_scale: float, tile_meta,
                              num_splits, causal: bool = True, out=None, lse=None, workspace=None):
    """The decode kernel of mla_decode_fp8_fwd alone (mla_combine_splits merges the split
    sequences' partials). Returns (out, lse, workspace)."""
    return _fp8_call("mla_decode_fp8_fwd_splits", q, kcodes, kscale, block_table, cache_seqlens, softmax_scale,
                     tile_meta, num_splits, causal, out, lse, workspace)


def _fp8_call(name, q, kcodes, kscale, block_table, cache_seqlens, softmax_scale, tile_meta, num_splits, causal, out,
              lse, workspace):
    import torch
    _need(q, torch.bfloat16, "q")
    dev = q.device
    _need(kcodes, torch.uint8, "kcodes", dev)
    _need(kscale, torch.float32, "kscale", dev)
    _need(block_table, torch.int32, "block_table", dev)
    _need(cache_seqlens, torch.int32, "cache_seqlens", dev)
    _need(tile_meta, torch.int32, "tile_meta", dev)
    _need(num_splits, torch.int32, "num_splits", dev)
    if q.dim() != 4 or q.shape[3] != D_QK:
        raise ValueError("q must be [B, s_q, h_q, 576]")
    if kcodes.dim() != 3 or kcodes.shape[1] != PAGE_SIZE or kcodes.shape[2] != D_QK:
        raise ValueError("kcodes must be [nblocks, 64, 576]")
    if tuple(kscale.shape) != tuple(kcodes.shape[:2]):
        raise ValueError("kscale must be [nblocks, 64]")
    B, s_q, h_q, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and cache_seqlens [B]")
    num_units = int(tile_meta.shape[0])
    with _on(torch, dev):
        if out is None:
            out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
        if workspace is None:
            ws = max(mla_fp8_plan_sizes(B, s_q, h_q)["workspace_bytes"], workspace_bytes(B, s_q, h_q, num_units))
            workspace = torch.empty((max(ws, 16),), dtype=torch.uint8, device=dev)
        _check(name, getattr(load_library(), name)(
            q.data_ptr(), kcodes.data_ptr(), kscale.data_ptr(), int(kcodes.shape[0]), block_table.data_ptr(),
            int(block_table.shape[1]), cache_seqlens.data_ptr(), B, s_q, h_q, float(softmax_scale),
            1 if causal else 0, tile_meta.data_ptr(), num_splits.data_ptr(), num_units, out.data_ptr(),
            lse.data_ptr(), workspace.data_ptr(), int(workspace.numel()), _stream(torch)))
    return out, lse, workspace


def mla_append_kv_fp8(kcodes, kscale, block_table, cache_seqlens, new_rows):
    """FP8 cache append: quantize new_rows bf16 [B, s_new, 576] into (kcodes, kscale) at
    positions cache_seqlens[b] - s_new + i. Updates both in place and returns them."""
    import torch
    _need(kcodes, torch.uint8, "kcodes")
    dev = kcodes.device
    _need(kscale, torch.float32, "kscale", dev)
    _need(block_table, torch.int32, "block_table", dev)
    _need(cache_seqlens, torch.int32, "cache_seqlens", dev)
    _need(new_rows, torch.bfloat16, "new_rows", dev)
    if kcodes.dim() != 3 or kcodes.shape[1] != PAGE_SIZE or kcodes.shape[2] != D_QK or \
            tuple(kscale.shape) != tuple(kcodes.shape[:2]):
        raise ValueError("kcodes must be [nblocks, 64, 576] and kscale [nblocks, 64]")
    if new_rows.dim() != 3 or new_rows.shape[2] != D_QK:
        raise ValueError("new_rows must be [B, s_new, 576]")
    B, s_new = int(new_rows.shape[0]), int(new_rows.shape[1])
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and cache_seqlens [B]")
    with _on(torch, dev):
        _check("mla_append_kv_fp8", load_library().mla_append_kv_fp8(
            kcodes.data_ptr(), kscale.data_ptr(), int(kcodes.shape[0]), block_table.data_ptr(),
            int(block_table.shape[1]), cache_seqlens.data_ptr(), new_rows.data_ptr(), B, s_new, _stream(torch)))
    return kcodes, kscale


def mla_append_kv(kcache, block_table, cache_seqlens, new_rows):
    """Cache append: new_rows bf16 [B, s_new, 576] go to token positions
    cache_seqlens[b] - s_new + i of their sequence (cache_seqlens counts them).
    kcache bf16 [nblocks, 64, 576] is updated in place and returned."""
    import torch
    _need(kcache, torch.bfloat16, "kcache")
    dev = kcache.device
    _need(block_table, torch.int32, "block_table", dev)
    _need(cache_seqlens, torch.int32, "cache_seqlens", dev)
    _need(new_rows, torch.bfloat16, "new_rows", dev)
    if kcache.dim() != 3 or kcache.shape[1] != PAGE_SIZE or kcache.shape[2] != D_QK:
        raise ValueError("kcache must be [nblocks, 64, 576]")
    if new_rows.dim() != 3 or new_rows.shape[2] != D_QK:
        raise ValueError("new_rows must be [B, s_new, 576]")
    B, s_new = int(new_rows.shape[0]), int(new_rows.shape[1])
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and cache_seqlens [B]")
    with _on(torch, dev):
        _check("mla_append_kv", load_library().mla_append_kv(
            kcache.data_ptr(), int(kcache.shape[0]), block_table.data_ptr(), int(block_table.shape[1]),
            cache_seqlens.data_ptr(), new_rows.data_ptr(), B, s_new, _stream(torch)))
    return kcache


class BlockPool:
    """Host bookkeeping of the paged cache's blocks (mla_block_pool_* in the
    library): per-slot block lists that grow and shrink, and the block tables
    the device calls take."""

    def __init__(self, nblocks: int, max_seqs: int, max_blocks_per_seq: int):
        self._lib = load_library()
        h = ctypes.c_void_p(None)
        _check("mla_block_pool_create", self._lib.mla_block_pool_create(int(nblocks), int(max_seqs),
                                                                        int(max_blocks_per_seq), ctypes.byref(h)))
        self._h = h
        self.nblocks, self.max_seqs, self.max_blocks_per_seq = int(nblocks), int(max_seqs), int(max_blocks_per_seq)

    def close(self):
        if self._h is not None and self._h.value:
            self._lib.mla_block_pool_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, seq: int, new_len: int):
        """Give slot seq room for new_len tokens (and make that its length)."""
        _check("mla_block_pool_reserve", self._lib.mla_block_pool_reserve(self._h, int(seq), int(new_len)))

    def release(self, seq: int):
        _check("mla_block_pool_release", self._lib.mla_block_pool_release(self._h, int(seq)))

    def free_blocks(self) -> int:
        return int(self._lib.mla_block_pool_free_blocks(self._h))

    def table(self, seqs, max_blocks: int):
        """(block_table int32 [n, max_blocks] padded with -1, lengths int32 [n]) as numpy arrays."""
        seqs = np.ascontiguousarray(np.asarray(seqs), dtype=np.int32)
        n = int(seqs.shape[0])
        table = np.zeros((n, int(max_blocks)), dtype=np.int32)
        lens = np.zeros((n,), dtype=np.int32)
        _check("mla_block_pool_table", self._lib.mla_block_pool_table(self._h, seqs.ctypes.data, n, int(max_blocks),
                                                                      table.ctypes.data, lens.ctypes.data))
        return table, lens


def workspace_bytes(batch: int, s_q: int, h_q: int, num_units: int) -> int:
    """Workspace mla_decode_fwd needs for a plan of num_units units (asks the library)."""
    n = ctypes.c_size_t(0)
    _check("mla_workspace_bytes", load_library().mla_workspace_bytes(batch, s_q, h_q, num_units, ctypes.byref(n)))
    return n.value


__all__ = ["mla_plan_sizes", "mla_workspace_bytes", "mla_get_metadata", "mla_get_metadata_host", "mla_decode_fwd",
           "mla_decode_fwd_splits", "mla_combine_splits", "mla_append_kv", "BlockPool",
           "mla_sparse_plan_sizes", "mla_get_metadata_sparse", "mla_decode_sparse_fwd",
           "mla_fp8_plan_sizes", "mla_get_metadata_fp8", "mla_decode_fp8_fwd", "mla_append_kv_fp8",
           "workspace_bytes", "load_library", "status_string", "MLAError", "LIB_PATH",
           "D_QK", "D_V", "PAGE_SIZE", "META_INTS", "mla_check_inputs_host", "mla_decode_sparse_fwd_splits",
           "mla_decode_fp8_fwd_splits"]
