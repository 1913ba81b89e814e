"""8-bit floating-point KV cache (oracle; test infrastructure).

Source: [PAG] Ultralytics glossary, "PagedAttention", "Related techniques": FP8
cache quantization keeps the cached keys and values at 8 bits, about half the
memory of a 16-bit cache.  The page names neither the 8-bit format nor how values
are scaled into it; the readings below fill that in.

Readings:
  R22 the format is the OCP 8-bit floating-point E4M3 encoding (1 sign bit, 4
      exponent bits with bias 7, 3 mantissa bits; no infinities; exponent 15 with
      mantissa 7 is NaN, so the largest finite magnitude is 448; exponent 0 holds
      the subnormals m * 2^-9).  Conversion rounds the magnitude to nearest, ties
      to the even code, saturates at 448 and keeps the sign bit (a negative value
      that rounds to zero becomes -0, code 0x80).
  R23 one float32 scale per cached row, i.e. per (token, KV head): with amax =
      max_c |x_c|, scale = amax / 448 is stored and code_c = E4M3(x_c * r) with
      r = 448 / amax; each of the two quotients and the product is rounded once
      in float32 (the kernel's precision, so both sides take the same rounding
      decision).  One division per row, one product per value.  A row whose
      amax is below 2^-112 (zero included; there 448 / amax would leave the
      float32 range) is stored as scale 0 and codes 0.  The stored value is
      code * scale.  A per-row scale lets a decode step append a token to a
      partly filled block without touching the rows already there.
  R24 the cache (compaction output and decode appends) is the only thing kept at
      8 bits; the prefill and the decode query stay at 16 bits, and the decode
      attention uses the values code * scale.

Everything here is plain numpy; the E4M3 value table is built from the field
definition above, and encoding picks the nearest table entry.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .paged import BLOCK

E4M3_MAX = 448.0
TINY_ROW = 2.0 ** -112     # rows below this largest magnitude are stored as zeros (R23)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each 8-bit code (float64; NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite magnitudes, in code order 0x00..0x7E (increasing)
_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest E4M3 code (ties to the even code), saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no place in the cache")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)   # the sign survives, also at zero


def quantize_rows(x) -> Tuple[np.ndarray, np.ndarray]:
    """x [..., d] (values a float32 holds exactly) -> (codes uint8 [..., d], scale float32 [...]).

    R23: scale = amax / 448, code = E4M3(x * (448 / amax)), every step rounded to float32.
    """
    x32 = np.asarray(x, dtype=np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("inputs must be exact in float32 (the cache is written from 16-bit values)")
    amax = np.max(np.abs(x32), axis=-1)
    live = amax >= np.float32(TINY_ROW)
    safe = np.where(live, amax, np.float32(1.0)).astype(np.float32)
    scale = np.where(live, safe / np.float32(E4M3_MAX), np.float32(0.0)).astype(np.float32)
    r = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    q = (x32 * r[..., None]).astype(np.float32)
    codes = e4m3_encode(q)
    codes[~live] = 0
    return codes, scale


def dequantize_rows(codes, scale) -> np.ndarray:
    """Stored values code * scale (float64)."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def compact_into_pool_fp8(k: np.ndarray, v: np.ndarray, keep: Optional[np.ndarray], table: Sequence[int],
                          pool_k: np.ndarray, pool_v: np.ndarray, scale_k: np.ndarray, scale_v: np.ndarray,
                          off: int = 0) -> None:
    """The compaction of the 16-bit cache with every written row quantized (R23).

    k, v [n][Hkv][d]; keep [Hkv][k_eff] or None; pools uint8 [blocks][Hkv][16][d];
    scales float32 [blocks][Hkv][16].  Row t of head h goes to slot off + t.
    """
    n, hkv, d = k.shape
    if keep is None:
        keep = np.tile(np.arange(n), (hkv, 1))
    for h in range(hkv):
        for t, i in enumerate(keep[h]):
            p = off + t
            b, s = table[p // BLOCK], p % BLOCK
            ck, sk = quantize_rows(k[i, h, :])
            cv, sv = quantize_rows(v[i, h, :])
            pool_k[b, h, s, :] = ck
            pool_v[b, h, s, :] = cv
            scale_k[b, h, s] = sk
            scale_v[b, h, s] = sv


def append_row_fp8(pool_k: np.ndarray, pool_v: np.ndarray, scale_k: np.ndarray, scale_v: np.ndarray,
                   table: Sequence[int], pos: int, new_k: np.ndarray, new_v: np.ndarray) -> None:
    """Decode append (R14) into the quantized cache: new_k, new_v [Hkv][d] go to slot pos."""
    b, s = table[pos // BLOCK], pos % BLOCK
    pool_k[b, :, s, :], scale_k[b, :, s] = quantize_rows(new_k)
    pool_v[b, :, s, :], scale_v[b, :, s] = quantize_rows(new_v)


def gather_rows_fp8(pool: np.ndarray, scale: np.ndarray, table: Sequence[int], length: int) -> np.ndarray:
    """Read a quantized sequence back through its table as values: [length][Hkv][d] float64."""
    out = []
    for p in range(length):
        b, s = table[p // BLOCK], p % BLOCK
        out.append(dequantize_rows(pool[b, :, s, :], scale[b, :, s]))
    return np.stack(out) if out else np.zeros((0,) + pool.shape[1:2] + pool.shape[3:])
