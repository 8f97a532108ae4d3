"""Reference for MLA decode over an FP8 latent cache.

TEST INFRASTRUCTURE ONLY (see the package docstring). No GPU code, no shared
helpers with the HIP library.

Sources: page "MLA 和 MHA 的 Kernel 区别" (the cache holds only the latent
row, which is what makes it cheap to store in fewer bits; its remarks on
quantising in the latent space) and the FlashMLA overview page (the paged
64-token cache). The number format is OCP FP8 E4M3 as published in the OCP
8-bit floating point specification: sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 is subnormal (value m/8 * 2^-6); the
pattern S.1111.111 is NaN; there are no infinities; the largest finite
magnitude is 448.

Readings where the pages leave it open:

* One FP32 scale per token for its 512 latent values: the stored value of
  latent coordinate d of token t is decode(byte[t, d]) * scale[t]. The
  64-value rotary part stays BF16 (it carries position, and is small).
* Decode over this cache is decode over the dequantised rows: every formula
  of the BF16 reference applies unchanged to the rows
  [decode(bytes) * scale ; rope].
* The quantiser (used to make test caches from real-valued rows) takes
  scale = amax / 448 over the token's 512 values (zero rows get scale 1)
  and rounds x / scale to the nearest E4M3 value, ties to the even
  mantissa, never overflowing past 448.
"""

from __future__ import annotations

import math

import numpy as np

from .mla_ref import mla_decode_ref_f64

E4M3_MAX = 448.0


def e4m3_value(byte: int) -> float:
    """The real value of one E4M3 byte (NaN for the NaN patterns)."""
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Elementwise E4M3 bytes (uint8) -> float64."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def quantize_e4m3_rows(rows: np.ndarray):
    """rows [N, 512] real -> (codes uint8 [N, 512], scale float32 [N]).

    scale = amax / 448 per row (1 for an all-zero row), then x / scale is
    rounded to the nearest finite E4M3 value, ties to even mantissa."""
    rows = np.asarray(rows, dtype=np.float64)
    amax = np.abs(rows).max(axis=1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    # the stored scale is FP32; quantise against exactly that value
    y = rows / scale.astype(np.float64)[:, None]
    finite = np.array([b for b in range(256) if not math.isnan(_E4M3_TABLE[b])])
    vals = _E4M3_TABLE[finite]
    order = np.argsort(vals, kind="stable")
    vals, codes_sorted = vals[order], finite[order]
    # drop the duplicate zero (0x80, -0) so every value appears once
    keep = np.ones(vals.size, dtype=bool)
    keep[(vals == 0.0) & (codes_sorted == 0x80)] = False
    vals, codes_sorted = vals[keep], codes_sorted[keep]
    idx = np.clip(np.searchsorted(vals, y), 1, vals.size - 1)
    lo, hi = vals[idx - 1], vals[idx]
    pick_hi = (hi - y) < (y - lo)
    tie = (hi - y) == (y - lo)
    even_hi = (codes_sorted[idx] & 1) == 0
    pick_hi = pick_hi | (tie & even_hi)
    out_idx = np.where(pick_hi, idx, idx - 1)
    out_idx = np.where(y >= vals[-1], vals.size - 1, out_idx)
    out_idx = np.where(y <= vals[0], 0, out_idx)
    return codes_sorted[out_idx].astype(np.uint8).reshape(rows.shape), scale


def dequantize_fp8_cache(latent_codes: np.ndarray, rope_bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP8 cache pieces -> float64 rows [num_pages, 64, 1, 576].

    latent_codes uint8 [P, 64, 512]; rope_bits uint16 (BF16) [P, 64, 64];
    scales float32 [P, 64]."""
    lat = e4m3_decode(latent_codes) * np.asarray(scales, dtype=np.float64)[..., None]
    rope = (np.asarray(rope_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    rows = np.concatenate([lat, rope.astype(np.float64)], axis=-1)
    return rows[:, :, None, :]


def mla_decode_fp8_ref(q_bits, latent_codes, rope_bits, scales, block_table, seqlens, scale, causal,
                       seqs=None):
    """Decode over the FP8 cache: the BF16 reference applied to the
    dequantised rows. q_bits uint16 [B, s_q, h_q, 576]."""
    q = (np.asarray(q_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    table = np.asarray(block_table)
    if seqs is not None:
        # dequantise only the pages the chosen sequences use (full-size caches)
        used = sorted({int(table[b, i]) for b in seqs for i in range((int(seqlens[b]) + 63) // 64)})
        remap = {page: k for k, page in enumerate(used)}
        table = table.copy()
        for b in seqs:
            for i in range((int(seqlens[b]) + 63) // 64):
                table[b, i] = remap[int(table[b, i])]
        latent_codes, rope_bits, scales = latent_codes[used], rope_bits[used], scales[used]
    kv = dequantize_fp8_cache(latent_codes, rope_bits, scales)
    return mla_decode_ref_f64(q.astype(np.float64), kv, table, seqlens,
                              float(np.float32(scale)), causal, seqs)
