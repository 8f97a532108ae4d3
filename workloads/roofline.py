"""Algorithmic work of one paged MLA decode call, and MI355X peak figures.

The byte count charges each cache row once: the query-key step and the
value step both read the same 576-value row, and the value step uses its
first 512 values (page "MLA 和 MHA 的 Kernel 区别", section on decode HBM
access: MLA reads ``seq_len x latent_dim`` once, versus MHA reading K and V).
Query, output, log-sum-exp, the used block-table entries and the lengths
are added. Split partials, metadata and re-reads are excluded on purpose:
they are implementation overheads and show up in the counter bytes instead.

The FLOP count is the two contractions only, 2*(576+512) per (row, visible
key) pair; exponentials and rescaling are not counted.
"""

from __future__ import annotations

import numpy as np

# Published MI355X peaks (datasheet): HBM3E bandwidth, dense BF16 MFMA.
MI355X_HBM_GBPS = 8000.0
MI355X_BF16_TFLOPS = 2500.0

_ROW_BYTES = 576 * 2
_OUT_BYTES = 512 * 2


def kv_read_bytes(seq_len: int, elems_per_token: int, bytes_per_elem: int = 2,
                  reads: int = 1) -> int:
    """Bytes read from a cache of ``seq_len`` tokens holding ``elems_per_token``
    values each, read ``reads`` times."""
    return int(seq_len) * int(elems_per_token) * int(bytes_per_elem) * int(reads)


def visible_lengths(seqlens, s_q: int, causal: bool) -> np.ndarray:
    """Keys visible to query token i of sequence b: N_b, or under the causal
    mask N_b - s_q + i + 1, clipped to [0, N_b]. Shape [B, s_q]."""
    n = np.asarray(seqlens, dtype=np.int64)[:, None]
    i = np.arange(s_q, dtype=np.int64)[None, :]
    if causal:
        return np.clip(n - s_q + i + 1, 0, n)
    return np.broadcast_to(n, (n.shape[0], s_q)).copy()


# FP8 cache row: 512 E4M3 latent bytes, 64 BF16 rotary values, one FP32 scale
_FP8_ROW_BYTES = 512 + 64 * 2 + 4


def algorithmic_bytes(seqlens, s_q: int, h_q: int, row_bytes: int = _ROW_BYTES) -> int:
    """`row_bytes` is what one cached token costs: 1152 for the BF16 cache,
    644 for the FP8 cache (``algorithmic_bytes_fp8``)."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    b = seqlens.size
    rows = b * s_q * h_q
    pages = int(((seqlens + 63) // 64).sum())
    return int(row_bytes * int(seqlens.sum()) + _ROW_BYTES * rows + _OUT_BYTES * rows
               + 4 * rows + 4 * pages + 4 * b)


def algorithmic_bytes_fp8(seqlens, s_q: int, h_q: int) -> int:
    return algorithmic_bytes(seqlens, s_q, h_q, _FP8_ROW_BYTES)


def algorithmic_flops(seqlens, s_q: int, h_q: int, causal: bool) -> int:
    lv = visible_lengths(seqlens, s_q, causal)
    return int(2 * (576 + 512) * h_q * int(lv.sum()))
