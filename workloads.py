"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds no attention arithmetic: it only draws sequence lengths, a shuffled block
table and normally distributed bf16 values, so that the HIP path and the CPU
oracle can be fed identical bytes.

Shapes follow the decode problem the FlashMLA pages describe (page 2, "Key
Highlights": BF16, paged KV cache with block size 64; page 4 release notes:
variable-length serving): queries q[B, s_q, h_q, 576], a block pool
kcache[nblocks, 64, 576] whose first 512 columns are also V, a block table
[B, max_blocks] and cache_seqlens[B].

Recipe (the same for every workload):
  1. cache_seqlens from the workload's length law, drawn first from
     numpy.random.default_rng(seed) (PCG64), seed = workload index.
  2. n_b = ceil(L_b / 64) blocks per sequence, nblocks = sum(n_b) + 4 spare
     blocks; physical ids = rng.permutation(nblocks) dealt to the sequences in
     order; block_table padded with -1 to max_b n_b columns.
  3. kcache = N(0,1) float32 rounded to bf16 (round to nearest even), then
     q = N(0,1) float32 rounded to bf16.
  4. With poison=True the cache rows that no sequence may read (rows >= L_b of
     a sequence's last block, and the spare blocks) hold bf16 NaN, so that any
     read of them shows up in the result.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D_QK = 576          # cached row width: 512 latent + 64 rope columns
D_V = 512           # V is the first 512 columns of the same row
PAGE = 64           # tokens per cache block
BF16_NAN = 0x7FC0

# name -> (index, description). The index is the RNG seed.
WORKLOADS = {
    "tiny": 0,
    "memory_bound": 1,
    "compute_bound": 2,
    "mixed": 3,
    "long": 4,
}

DESCRIPTIONS = {
    "tiny": "B=2, cache_seqlens {64,200}, s_q=1, h_q=16",
    "memory_bound": "B=16, cache_seqlens U[1024,4096], s_q=1, h_q=16",
    "compute_bound": "B=64, cache_seqlens 4096, s_q=1, h_q=128",
    "mixed": "B=128, cache_seqlens log-U[256,16384], s_q=2 causal, h_q=128",
    "long": "B=8, cache_seqlens 32768, s_q=1, h_q=16",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class DecodeInputs:
    """One decode batch. Arrays are host numpy; bf16 tensors are uint16 bit patterns."""
    name: str
    q: np.ndarray               # uint16 [B, s_q, h_q, 576]
    kcache: np.ndarray          # uint16 [nblocks, 64, 576]
    block_table: np.ndarray     # int32  [B, max_blocks]
    cache_seqlens: np.ndarray   # int32  [B]
    s_q: int
    h_q: int
    softmax_scale: float
    causal: bool
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.cache_seqlens.shape[0])


def _seqlens(name: str, rng: np.random.Generator) -> np.ndarray:
    if name == "tiny":
        return np.array([64, 200], dtype=np.int32)
    if name == "memory_bound":
        return rng.integers(1024, 4097, 16).astype(np.int32)
    if name == "compute_bound":
        return np.full(64, 4096, dtype=np.int32)
    if name == "mixed":
        x = np.exp(rng.uniform(math.log(256.0), math.log(16384.0), 128))
        return np.clip(np.round(x), 256, 16384).astype(np.int32)
    if name == "long":
        return np.full(8, 32768, dtype=np.int32)
    raise KeyError(name)


def _shape(name: str):
    """(s_q, h_q, causal) of a named workload."""
    return {
        "tiny": (1, 16, True),
        "memory_bound": (1, 16, True),
        "compute_bound": (1, 128, True),
        "mixed": (2, 128, True),
        "long": (1, 16, True),
    }[name]


def build_inputs(seqlens, s_q: int, h_q: int, rng: np.random.Generator, *,
                 name: str = "custom", causal: bool = True, poison: bool = True,
                 softmax_scale: float = 1.0 / math.sqrt(192.0), spare_blocks: int = 4,
                 d_qk: int = D_QK, page: int = PAGE) -> DecodeInputs:
    """Draw a paged cache, block table and queries for the given sequence lengths."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    B = int(seqlens.shape[0])
    nb = (seqlens.astype(np.int64) + page - 1) // page
    nblocks = int(nb.sum()) + spare_blocks
    max_blocks = max(int(nb.max()) if B else 0, 1)
    perm = rng.permutation(nblocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nb[b])
        table[b, :n] = perm[off:off + n]
        off += n
    kcache = f32_to_bf16_bits(rng.standard_normal((nblocks, page, d_qk), dtype=np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((B, s_q, h_q, d_qk), dtype=np.float32))
    if poison:
        used = np.zeros(nblocks, dtype=bool)
        for b in range(B):
            n = int(nb[b])
            used[table[b, :n]] = True
            tail = int(seqlens[b]) - (n - 1) * page if n else page
            if n and tail < page:
                kcache[table[b, n - 1], tail:, :] = BF16_NAN
        kcache[~used] = BF16_NAN
    return DecodeInputs(name=name, q=q, kcache=kcache, block_table=table,
                        cache_seqlens=seqlens, s_q=s_q, h_q=h_q,
                        softmax_scale=float(softmax_scale), causal=causal,
                        meta={"nblocks": nblocks, "max_blocks": max_blocks, "poison": poison})


def make_workload(name: str, *, poison: bool = True) -> DecodeInputs:
    """The named workload, seeded with its index."""
    seed = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    lens = _seqlens(name, rng)
    s_q, h_q, causal = _shape(name)
    return build_inputs(lens, s_q, h_q, rng, name=name, causal=causal, poison=poison)


def subset(inp: DecodeInputs, batch_idx) -> DecodeInputs:
    """The same cache with only the sequences batch_idx (rows of q/table/lens kept in order)."""
    batch_idx = np.asarray(batch_idx, dtype=np.int64)
    return DecodeInputs(name=inp.name + "[sub]", q=np.ascontiguousarray(inp.q[batch_idx]),
                        kcache=inp.kcache, block_table=np.ascontiguousarray(inp.block_table[batch_idx]),
                        cache_seqlens=np.ascontiguousarray(inp.cache_seqlens[batch_idx]),
                        s_q=inp.s_q, h_q=inp.h_q, softmax_scale=inp.softmax_scale,
                        causal=inp.causal, meta=dict(inp.meta))


def visible_tokens(seqlens, s_q: int, causal: bool) -> np.ndarray:
    """Tokens each query position sees: [B, s_q] (new tokens are the last s_q cached positions)."""
    L = np.asarray(seqlens, dtype=np.int64)[:, None]
    i = np.arange(s_q, dtype=np.int64)[None, :]
    v = L - (s_q - 1 - i) if causal else np.broadcast_to(L, (L.shape[0], s_q))
    return np.clip(v, 0, None)


def algorithmic_counts(seqlens, s_q: int, h_q: int, causal: bool,
                       d_qk: int = D_QK, d_v: int = D_V, page: int = PAGE):
    """Bytes and FLOPs the method must move/compute, each cached row counted once.

    bytes = sum_b L_b * 2*d_qk  (cache rows)
          + B*s_q*h_q*(2*d_qk + 2*d_v + 4)  (q in, out bf16 and lse fp32 out)
          + 4*sum_b n_b + 4*B  (block table entries used, cache_seqlens)
    flops = sum_b sum_i h_q * 2 * V(b,i) * (d_qk + d_v)   (QK^T and PV MACs)
    """
    L = np.asarray(seqlens, dtype=np.int64)
    B = L.shape[0]
    nb = (L + page - 1) // page
    nbytes = int(L.sum()) * 2 * d_qk + B * s_q * h_q * (2 * d_qk + 2 * d_v + 4) + 4 * int(nb.sum()) + 4 * B
    vis = visible_tokens(L, s_q, causal)
    flops = int(vis.sum()) * h_q * 2 * (d_qk + d_v)
    return nbytes, flops



def fp8_counts(seqlens, s_q: int, h_q: int, causal: bool, d_qk: int = D_QK, d_v: int = D_V, page: int = PAGE):
    """Algorithmic (bytes, flops) of a decode over the FP8 cache: as algorithmic_counts,
    but each cached row is d_qk one-byte codes plus its 4-byte float32 scale."""
    L = np.asarray(seqlens, dtype=np.int64)
    B = L.shape[0]
    nb = (L + page - 1) // page
    nbytes = int(L.sum()) * (d_qk + 4) + B * s_q * h_q * (2 * d_qk + 2 * d_v + 4) + 4 * int(nb.sum()) + 4 * B
    flops = int(visible_tokens(L, s_q, causal).sum()) * h_q * 2 * (d_qk + d_v)
    return nbytes, flops


def rows_in_token_order(inp: DecodeInputs) -> np.ndarray:
    """uint16 [B, max_L, d_qk]: sequence b's cached rows in token order, right-aligned
    (row i holds token L_b - max_L + i; rows before token 0 are zero)."""
    L = inp.cache_seqlens.astype(np.int64)
    B = L.shape[0]
    T = int(L.max()) if B else 0
    page = inp.kcache.shape[1]
    rows = np.zeros((B, T, inp.kcache.shape[2]), dtype=np.uint16)
    for b in range(B):
        t = np.arange(int(L[b]))
        rows[b, T - int(L[b]):] = inp.kcache[inp.block_table[b, t // page], t % page]
    return rows


# ---------------------------------------------------------------- cache append

APPEND_SEED = 11
APPEND_DESCRIPTION = "B=64 sequences, 512 new tokens each, cache_seqlens U[1024,4096] after the append"


@dataclass
class AppendInputs:
    """One cache-append batch (host numpy; bf16 as uint16 bits)."""
    kcache: np.ndarray          # uint16 [nblocks, 64, 576]
    block_table: np.ndarray     # int32  [B, max_blocks]
    cache_seqlens: np.ndarray   # int32  [B], lengths including the new tokens
    new_rows: np.ndarray        # uint16 [B, s_new, 576]


def make_append(batch: int = 64, s_new: int = 512, seed: int = APPEND_SEED) -> AppendInputs:
    """Lengths U[1024, 4096] after the append, a shuffled block table as for the
    decode workloads, an N(0,1) cache and N(0,1) new rows, seeded."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 4097, batch).astype(np.int32)
    nb = (lens + PAGE - 1) // PAGE
    nblocks = int(nb.sum()) + 4
    perm = rng.permutation(nblocks).astype(np.int32)
    table = np.full((batch, int(nb.max())), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    kcache = f32_to_bf16_bits(rng.standard_normal((nblocks, PAGE, D_QK), dtype=np.float32))
    new_rows = f32_to_bf16_bits(rng.standard_normal((batch, s_new, D_QK), dtype=np.float32))
    return AppendInputs(kcache=kcache, block_table=table, cache_seqlens=lens, new_rows=new_rows)


def append_bytes(inp: AppendInputs, fp8: bool = False) -> int:
    """Algorithmic HBM bytes of one append: every new row read once (bf16) and written
    once (bf16, or for the FP8 cache its codes and its 4-byte scale), plus the
    block-table entries and lengths the kernel reads."""
    B, s_new, width = inp.new_rows.shape
    rows = int(np.minimum(inp.cache_seqlens, s_new).sum())
    written = width + 4 if fp8 else 2 * width
    return rows * (2 * width + written) + 4 * rows + 4 * B


# ---------------------------------------------------------------- sparse decode

SPARSE_SEED = 12
SPARSE_DESCRIPTION = ("B=64, s_q=1, h_q=16, topk=2048 distinct positions drawn uniformly from [0, L), "
                      "cache_seqlens U[4096,16384]")


@dataclass
class SparseInputs:
    """One sparse-decode batch (host numpy; bf16 as uint16 bits)."""
    dec: DecodeInputs           # q, kcache, block_table, cache_seqlens (non-causal)
    indices: np.ndarray         # int32 [B, s_q, topk]
    counts: np.ndarray          # int32 [B * s_q]


def make_sparse(batch: int = 64, s_q: int = 1, h_q: int = 16, topk: int = 2048, lo: int = 4096, hi: int = 16384,
                seed: int = SPARSE_SEED, poison: bool = False) -> SparseInputs:
    """Lengths U[lo, hi], the decode recipe for the cache and queries, then for
    every new token topk distinct positions of its sequence, uniformly drawn."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, batch).astype(np.int32)
    dec = build_inputs(lens, s_q, h_q, rng, name="sparse", causal=False, poison=poison)
    idx = np.empty((batch, s_q, topk), dtype=np.int32)
    for b in range(batch):
        for i in range(s_q):
            idx[b, i] = rng.choice(int(lens[b]), size=topk, replace=False)
    counts = np.full((batch * s_q,), topk, dtype=np.int32)
    return SparseInputs(dec=dec, indices=idx, counts=counts)


def sparse_counts(inp: SparseInputs):
    """Algorithmic (bytes, flops) of one sparse decode: each listed row once per
    new token (1152 B), q, out, lse and the list entries; 2*h*(576+512) flops
    per listed row and head."""
    d = inp.dec
    B, s_q, h_q = d.batch, d.s_q, d.h_q
    valid = int((inp.indices >= 0).sum())
    nbytes = valid * D_QK * 2 + B * s_q * h_q * (D_QK * 2 + D_V * 2 + 4) + 4 * inp.indices.size + 4 * B * s_q
    flops = 2 * h_q * (D_QK + D_V) * valid
    return nbytes, flops
