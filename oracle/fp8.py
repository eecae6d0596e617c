"""FP8 (E4M3) row quantizer for the latent cache (test infrastructure).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this module; it shares nothing with the HIP library.

The FlashMLA explainer (theflyingbirds.in) lists FP8 support under section 9,
"Future Directions", to cut memory further; the pages fix no format. Reading
taken (listed in the design notes): OCP E4M3 codes (bias 7, subnormals, no
infinities, 0x7F/0xFF NaN), one float32 scale per cached row covering its
576 columns, chosen so the row's largest magnitude maps to 448, the largest
E4M3 value:
    amax  = max_d |x_d|                (exact: bf16 values widened to float32)
    scale = amax / 448                 (float32 division)
    code  = E4M3 nearest to x_d * (448 / amax), ties to the even code
            (the quotient and the product each rounded to float32)
    a row of zeros gets scale 0 and codes 0.
Decoding is code value * scale.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF), from the format definition."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_VALS = e4m3_table()
_POS = np.array([c for c in range(128) if not np.isnan(_VALS[c])], dtype=np.int64)   # 0x00..0x7E, increasing


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """uint8 codes of float32 values |x| <= 448: nearest value, ties to the even code."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    mag = np.abs(x)
    vals = _VALS[_POS]
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_hi = np.abs(vals[hi] - mag)
    d_lo = np.abs(mag - vals[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS[hi] & 1) == 0))
    code = np.where(pick_hi, _POS[hi], _POS[lo]).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(rows_bf16_bits: np.ndarray):
    """rows uint16 bf16 bits [..., width] -> (codes uint8 [..., width], scales float32 [...])."""
    x = (np.ascontiguousarray(rows_bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(0), (safe / np.float32(E4M3_MAX)).astype(np.float32)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    codes = round_to_e4m3(y)
    codes = np.where(zero[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values code * scale."""
    return _VALS[codes] * np.asarray(scales, dtype=np.float64)[..., None]


def append_rows_fp8(codes, scales, block_table, cache_seqlens, new_rows_bf16, page: int = 64):
    """The FP8 cache append: quantize the new rows, then write code rows and
    scales at positions cache_seqlens[b] - s_new + i (negative ones skipped)."""
    qc, qs = quantize_rows(new_rows_bf16)
    codes = np.array(codes, copy=True)
    scales = np.array(scales, copy=True)
    B, s_new = new_rows_bf16.shape[0], new_rows_bf16.shape[1]
    for b in range(B):
        length = int(cache_seqlens[b])
        for i in range(s_new):
            pos = length - s_new + i
            if pos < 0:
                continue
            blk = int(block_table[b, pos // page])
            codes[blk, pos % page, :] = qc[b, i]
            scales[blk, pos % page] = qs[b, i]
    return codes, scales
