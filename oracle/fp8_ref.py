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
* The quantiser (the cache writer's rule) stores one FP32 scale per token,
  the FP32 number nearest amax / 448 over the token's 512 values (zero rows
  get scale 1), and codes each value as the E4M3 value nearest the exact
  quotient x / scale, ties to the even mantissa, saturating at 448. That is
  the format's round-to-nearest applied to the real number the stored
  scale and the input define; no intermediate rounding of the quotient
  enters the definition.
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
    """rows [N, 512] (values exact in float32, e.g. BF16 inputs) ->
    (codes uint8 [N, 512], scale float32 [N]).

    The scale is stored as an FP32 number: scale = fl32(amax / 448), the
    FP32 value nearest the row's largest magnitude over 448 (1 for an
    all-zero row). Each value's code is the E4M3 value nearest the exact
    quotient |x| / scale, ties to the even mantissa, magnitudes past 448
    saturating to 448; the sign bit is x's (a negative value that rounds to
    zero gives 0x80, negative zero).

    The nearest grid value is found by counting the midpoints between
    neighbouring grid values that lie strictly below the quotient; a
    quotient exactly at a midpoint takes the even code of the two. Each
    comparison |x| > mid * scale is exact in float64: mid has at most five
    significant bits and scale 24, so their product is a float64 number."""
    x = np.asarray(rows, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    grid = _E4M3_TABLE[:0x7F]                      # codes 0x00..0x7E, increasing
    mids = (grid[:-1] + grid[1:]) / 2              # 126 midpoints, exact in float64
    odd = (np.arange(mids.size) % 2) == 1          # midpoint k lies between codes k and k + 1
    mag = np.abs(x).astype(np.float64)
    code = np.empty(x.shape, dtype=np.int64)
    for r in range(x.shape[0]):
        bounds = mids * float(scale[r])            # exact products, increasing
        below = np.searchsorted(bounds, mag[r], side="left")   # midpoints strictly below
        at = np.zeros(mag.shape[1], dtype=bool)
        inside = below < bounds.size
        at[inside] = bounds[below[inside]] == mag[r, inside]
        code[r] = below + (at & odd[np.minimum(below, bounds.size - 1)])
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8), scale


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


def kv_append_fp8_ref(latent_codes, rope_bits, scales, new_bits, block_table, seqlens):
    """Append into an FP8 cache: the placement of ``kv_append_ref`` (token i
    of a sequence holding N tokens after the append goes to position
    N - s_new + i; negative positions dropped, missing pages counted), each
    placed token's latent part quantised by ``quantize_e4m3_rows`` and its
    rotary part copied. Returns (codes, rope, scales, skipped), new arrays."""
    codes = np.array(latent_codes, copy=True)
    rope = np.array(rope_bits, copy=True)
    sc = np.array(scales, copy=True)
    bsz, s_new, _ = new_bits.shape
    width = block_table.shape[1]
    x = (np.asarray(new_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    skipped = 0
    for b in range(bsz):
        n = int(seqlens[b])
        for i in range(s_new):
            pos = n - s_new + i
            if pos < 0:
                continue
            logical = pos // 64
            page = int(block_table[b, logical]) if logical < width else -1
            if page < 0 or page >= codes.shape[0]:
                skipped += 1
                continue
            q, s1 = quantize_e4m3_rows(x[b, i:i + 1, :512])
            codes[page, pos % 64] = q[0]
            sc[page, pos % 64] = s1[0]
            rope[page, pos % 64] = new_bits[b, i, 512:]
    return codes, rope, sc, skipped
