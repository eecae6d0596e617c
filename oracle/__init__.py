"""CPU oracle for MLA decode over a paged latent cache (test infrastructure).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. It builds oracle/mla_oracle.c with gcc into oracle/_build and
calls it through ctypes. It shares nothing with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "mla_oracle.c"
_SRC_SPARSE = _HERE / "mla_oracle_sparse.c"
_SRC_FP8 = _HERE / "mla_oracle_fp8.c"
_BUILD = _HERE / "_build"
_LIB = _BUILD / "liboracle.so"
_lib = None


def build(force: bool = False, src=None, out: Path = _LIB) -> Path:
    """Compile the oracle with gcc (no GPU code, no HIP headers). src: one C
    file or a list of them (default: the dense, sparse and FP8 decode oracles)."""
    srcs = [_SRC, _SRC_SPARSE, _SRC_FP8] if src is None else ([src] if isinstance(src, (str, Path)) else list(src))
    srcs = [Path(x) for x in srcs]
    out.parent.mkdir(parents=True, exist_ok=True)
    if force or not out.exists() or any(out.stat().st_mtime < x.stat().st_mtime for x in srcs):
        tmp = out.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        *[str(x) for x in srcs], "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, out)
    return out


def load(path: Path | None = None):
    """Load (building first if needed) and return the ctypes handle."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(str(path))
    else:
        if _lib is not None:
            return _lib
        alt = os.environ.get("MLA_ORACLE_LIB")    # a sanitizer build of the same sources (tests)
        if alt:
            lib = ctypes.CDLL(alt)
        else:
            build()
            lib = ctypes.CDLL(str(_LIB))
    fn = lib.mla_oracle_decode
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    if hasattr(lib, "mla_oracle_decode_sparse"):
        sp = lib.mla_oracle_decode_sparse
        sp.restype = ctypes.c_int
        sp.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 8 + [ctypes.c_double, ctypes.c_void_p,
                                                                     ctypes.c_void_p, ctypes.c_int]
    if hasattr(lib, "mla_oracle_decode_fp8"):
        f8 = lib.mla_oracle_decode_fp8
        f8.restype = ctypes.c_int
        f8.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                                                     ctypes.c_void_p, ctypes.c_int]
        lib.mla_oracle_e4m3_value.restype = ctypes.c_double
        lib.mla_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    if path is None:
        _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def mla_decode(q, kcache, block_table, cache_seqlens, softmax_scale, causal=True,
               nthreads: int | None = None, d_v: int = 512, lib=None):
    """Oracle decode.

    q: uint16 bf16 bits [B, s_q, h_q, d_qk]; kcache: uint16 [nblocks, page, d_qk];
    block_table: int32 [B, max_blocks]; cache_seqlens: int32 [B].
    Returns (out float64 [B, s_q, h_q, d_v], lse float64 [B, s_q, h_q]).
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kcache = np.ascontiguousarray(kcache, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    cache_seqlens = np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    B, s_q, h_q, d_qk = q.shape
    nblocks, page, d_k2 = kcache.shape
    if d_k2 != d_qk:
        raise ValueError("q and kcache widths differ")
    if block_table.ndim != 2 or block_table.shape[0] != B or cache_seqlens.shape != (B,):
        raise ValueError("block_table / cache_seqlens shape mismatch")
    max_blocks = block_table.shape[1]
    out = np.zeros((B, s_q, h_q, d_v), dtype=np.float64)
    lse = np.zeros((B, s_q, h_q), dtype=np.float64)
    lib = lib or load()
    rc = lib.mla_oracle_decode(q.ctypes.data, kcache.ctypes.data, block_table.ctypes.data,
                               cache_seqlens.ctypes.data, B, s_q, h_q, max_blocks,
                               d_qk, d_v, page, float(softmax_scale), 1 if causal else 0,
                               out.ctypes.data, lse.ctypes.data,
                               int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle failed (%d)" % rc)
    return out, lse


def decode_inputs(inp, nthreads: int | None = None, lib=None):
    """Oracle decode of a workloads.DecodeInputs."""
    return mla_decode(inp.q, inp.kcache, inp.block_table, inp.cache_seqlens,
                      inp.softmax_scale, inp.causal, nthreads=nthreads, lib=lib)


def mla_decode_sparse(q, kcache, block_table, indices, counts, softmax_scale, nthreads: int | None = None,
                      d_v: int = 512, lib=None):
    """Oracle sparse decode: query row (b, i, h) attends over the tokens
    indices[b, i, :counts[b*s_q+i]] (entries < 0 skipped).

    q uint16 [B, s_q, h_q, d_qk]; kcache uint16 [nblocks, page, d_qk];
    block_table int32 [B, max_blocks]; indices int32 [B, s_q, topk];
    counts int32 [B * s_q]. Returns (out float64 [B, s_q, h_q, d_v], lse float64 [B, s_q, h_q]).
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kcache = np.ascontiguousarray(kcache, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    counts = np.ascontiguousarray(np.asarray(counts).reshape(-1), dtype=np.int32)
    B, s_q, h_q, d_qk = q.shape
    nblocks, page, _ = kcache.shape
    if indices.ndim != 3 or indices.shape[:2] != (B, s_q) or counts.shape != (B * s_q,):
        raise ValueError("indices must be [B, s_q, topk] and counts [B * s_q]")
    topk = indices.shape[2]
    out = np.zeros((B, s_q, h_q, d_v), dtype=np.float64)
    lse = np.zeros((B, s_q, h_q), dtype=np.float64)
    lib = lib or load()
    rc = lib.mla_oracle_decode_sparse(q.ctypes.data, kcache.ctypes.data, block_table.ctypes.data,
                                      indices.ctypes.data, counts.ctypes.data, B, s_q, h_q,
                                      block_table.shape[1], topk, d_qk, d_v, page, float(softmax_scale),
                                      out.ctypes.data, lse.ctypes.data, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("sparse oracle failed (%d)" % rc)
    return out, lse


def mla_decode_fp8(q, codes, scales, block_table, cache_seqlens, softmax_scale, causal=True,
                   nthreads: int | None = None, d_v: int = 512, lib=None):
    """Oracle decode over an FP8 cache: codes uint8 [nblocks, page, d_qk] (E4M3),
    scales float32 [nblocks, page]; otherwise as mla_decode."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    cache_seqlens = np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    B, s_q, h_q, d_qk = q.shape
    nblocks, page, width = codes.shape
    if width != d_qk or scales.shape != (nblocks, page):
        raise ValueError("codes must be [nblocks, page, d_qk] and scales [nblocks, page]")
    out = np.zeros((B, s_q, h_q, d_v), dtype=np.float64)
    lse = np.zeros((B, s_q, h_q), dtype=np.float64)
    lib = lib or load()
    rc = lib.mla_oracle_decode_fp8(q.ctypes.data, codes.ctypes.data, scales.ctypes.data, block_table.ctypes.data,
                                   cache_seqlens.ctypes.data, B, s_q, h_q, block_table.shape[1], d_qk, d_v, page,
                                   float(softmax_scale), 1 if causal else 0, out.ctypes.data, lse.ctypes.data,
                                   int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("fp8 oracle failed (%d)" % rc)
    return out, lse
