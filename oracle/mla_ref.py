"""FP64 reference for MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY (see the package docstring). No GPU code, no shared
helpers with the HIP library.

Sources (web pages, cited by title and section):

* FlashMLA overview page (nullthought.net, "FlashMLA Overview"): the decode
  kernel takes BF16 inputs, a paged KV cache with 64-token blocks, and
  variable-length sequences.
* "MLA 和 MHA 的 Kernel 区别" (MLA vs MHA kernel differences), section
  "内存布局和 KV Cache 大小" / MLA: the cache stores only the compressed
  vector c_KV; keys and values are up-projections of it, K = c_KV W_UK and
  V = c_KV W_UV.
* Same page, section "Decode 阶段的 HBM 访问模式" / "MLA Decode": for the
  new token, score every cached token, take the softmax of the scores, then
  sum the value vectors weighted by the softmax.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* Absorbed form. The query handed to decode has W_UK already folded in, so
  keys are the cache rows themselves, and the value vectors are the latent
  part of the same rows (W_UV is applied after decode). The non-absorbed
  form of the MLA page is kept here too (``mla_nonabsorbed_ref``) so a test
  can show both give the same answer.
* Each cache row has 576 values: 512 latent plus a 64-value rotary part that
  enters the scores only. The rotary part is already applied.
* Softmax scale is an input; the pages give none. It is taken exactly as the
  float32 value the GPU receives.
* ``lse`` is the natural log of the sum of exp(score) over visible keys.
* Causal mask for s_q new tokens: the new tokens' rows are already in the
  cache at its end, so token i sees keys t < N - s_q + i + 1.
* A row that sees no key outputs zeros and lse = -inf.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

PAGE = 64        # tokens per page (FlashMLA overview: block size 64)
D_QK = 576       # 512 latent + 64 rotary
D_V = 512        # latent part of the row


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float64. Exact: a BF16 value is the upper 16 bits
    of a float32, and float32 -> float64 is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def gather_sequence_rows(kv: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Logical cache rows of one sequence: row t lives in physical page
    ``table_row[t // 64]`` at slot ``t % 64`` (paged cache, block 64).

    ``kv`` is [num_pages, 64, 1, 576]; returns [n, 576]. Only the first
    ceil(n/64) table entries are read."""
    if n == 0:
        return np.zeros((0, kv.shape[-1]), dtype=kv.dtype)
    t = np.arange(n)
    pages = np.asarray(table_row)[t // PAGE]
    return kv[pages, t % PAGE, 0, :]


def visible_length(n: int, s_q: int, i: int, causal: bool) -> int:
    """Number of leading keys query token i of a sequence of n cached tokens
    may attend to."""
    if not causal:
        return n
    return max(0, min(n, n - s_q + i + 1))


def attend_rows(q: np.ndarray, k: np.ndarray, lengths: Sequence[int], scale: float):
    """Softmax attention of query rows over the leading keys, two passes.

    q: [R, 576]; k: [N, 576] (values are k[:, :512]); lengths[r] keys are
    visible to row r. Returns out [R, 512], lse [R] (float64).

    Rows that see the same keys (the same length L) are taken together.
    Pass 1 scores their visible keys, s_t = scale * <q, k_t> for t < L, and
    reduces each row to its log-sum-exp. Pass 2 weights the value rows by
    exp(s_t - lse) and sums them.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    r_count = q.shape[0]
    out = np.zeros((r_count, D_V), dtype=np.float64)
    lse = np.full(r_count, -np.inf, dtype=np.float64)
    lengths = np.asarray(lengths, dtype=np.int64).reshape(r_count)
    for L in np.unique(lengths):
        if L == 0:
            continue
        rows = np.nonzero(lengths == L)[0]
        keys = k[:L]
        s = scale * (q[rows] @ keys.T)             # [rows, L]
        m = s.max(axis=1)
        row_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        lse[rows] = row_lse
        out[rows] = np.exp(s - row_lse[:, None]) @ keys[:, :D_V]
    return out, lse


def mla_decode_ref_f64(q: np.ndarray, kv: np.ndarray, block_table: np.ndarray,
                       seqlens: np.ndarray, scale: float, causal: bool,
                       seqs: Optional[Sequence[int]] = None):
    """MLA decode over a paged cache, all in float64.

    q: [B, s_q, h_q, 576]; kv: [num_pages, 64, 1, 576];
    block_table: [B, max_blocks]; seqlens: [B].
    Returns out [B, s_q, h_q, 512] and lse [B, s_q, h_q]; with ``seqs`` only
    those sequences are computed (the rest stay zero / -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, s_q, h_q, _ = q.shape
    out = np.zeros((bsz, s_q, h_q, D_V), dtype=np.float64)
    lse = np.full((bsz, s_q, h_q), -np.inf, dtype=np.float64)
    for b in (range(bsz) if seqs is None else seqs):
        n = int(seqlens[b])
        k = gather_sequence_rows(kv, block_table[b], n)
        rows = q[b].reshape(s_q * h_q, D_QK)
        lengths = [visible_length(n, s_q, i, causal) for i in range(s_q) for _ in range(h_q)]
        o, l = attend_rows(rows, k, lengths, scale)
        out[b] = o.reshape(s_q, h_q, D_V)
        lse[b] = l.reshape(s_q, h_q)
    return out, lse


def mla_decode_ref(q_bits: np.ndarray, kv_bits: np.ndarray, block_table: np.ndarray,
                   seqlens: np.ndarray, scale: float, causal: bool,
                   seqs: Optional[Sequence[int]] = None):
    """``mla_decode_ref_f64`` on BF16 bit-pattern inputs. The scale is taken
    as the float32 value a caller passes to the GPU."""
    scale64 = float(np.float32(scale))
    if seqs is None:
        kv = bf16_bits_to_f64(kv_bits)
    else:
        # Convert only the pages the chosen sequences touch (full-size inputs).
        kv = _LazyPages(kv_bits)
    return mla_decode_ref_f64(bf16_bits_to_f64(q_bits), kv, block_table, seqlens,
                              scale64, causal, seqs)


class _LazyPages:
    """Indexable view that converts only the requested pages to float64."""

    def __init__(self, kv_bits):
        self._bits = kv_bits
        self.shape = kv_bits.shape
        self.dtype = np.float64

    def __getitem__(self, idx):
        pages, slots, head, cols = idx
        return bf16_bits_to_f64(self._bits[pages, slots, head, cols])


def lse_combine_ref(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge attention results computed over disjoint key subsets.

    o_parts[s] is the softmax-weighted value sum over subset s (normalised
    within the subset) and lse_parts[s] its log-sum-exp. The whole-set
    result is lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
    Subsets with lse_s = -inf carry no weight; if all are -inf the result is
    zeros and -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    total = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, total, 1.0)), -np.inf)
    weight = np.where(finite, w / np.where(finite, total, 1.0), 0.0)
    o = (weight[..., None] * o_parts).sum(axis=0)
    return o, lse


def mla_nonabsorbed_ref(c_kv: np.ndarray, k_rope: np.ndarray, q_nope: np.ndarray,
                        q_rope: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                        scale: float):
    """MLA decode for one token in the non-absorbed form of the MLA page
    ("MLA Decode" pseudo-code and the MLA projections): each cached latent
    row is up-projected per head, K_h = c_KV W_UK_h and V_h = c_KV W_UV_h,
    the head's score adds the rotary part, and the output is the
    softmax-weighted sum of V_h.

    c_kv [N, 512]; k_rope [N, 64]; q_nope [H, dn]; q_rope [H, 64];
    w_uk [H, 512, dn]; w_uv [H, 512, dv]. Returns o [H, dv], lse [H].
    """
    h_count = q_nope.shape[0]
    dv = w_uv.shape[2]
    o = np.zeros((h_count, dv))
    lse = np.zeros(h_count)
    for h in range(h_count):
        k_h = c_kv @ w_uk[h]                          # [N, dn]
        v_h = c_kv @ w_uv[h]                          # [N, dv]
        s = scale * (k_h @ q_nope[h] + k_rope @ q_rope[h])
        m = s.max()
        lse[h] = m + math.log(np.exp(s - m).sum())
        o[h] = np.exp(s - lse[h]) @ v_h
    return o, lse


def mla_decode_bruteforce(q: np.ndarray, kv: np.ndarray, block_table, seqlens,
                          scale: float, causal: bool):
    """The same definition in pure Python with exactly rounded sums
    (math.fsum), for tiny inputs. q and kv are float64 arrays."""
    bsz, s_q, h_q, _ = q.shape
    out = [[[[0.0] * D_V for _ in range(h_q)] for _ in range(s_q)] for _ in range(bsz)]
    lse = [[[-math.inf] * h_q for _ in range(s_q)] for _ in range(bsz)]
    for b in range(bsz):
        n = int(seqlens[b])
        keys = []
        for t in range(n):
            page = int(block_table[b][t // PAGE])
            keys.append([float(x) for x in kv[page][t % PAGE][0]])
        for i in range(s_q):
            L = visible_length(n, s_q, i, causal)
            for h in range(h_q):
                if L == 0:
                    continue
                qv = [float(x) for x in q[b][i][h]]
                s = [scale * math.fsum(qv[d] * keys[t][d] for d in range(D_QK)) for t in range(L)]
                m = max(s)
                ll = m + math.log(math.fsum(math.exp(x - m) for x in s))
                lse[b][i][h] = ll
                p = [math.exp(x - ll) for x in s]
                out[b][i][h] = [math.fsum(p[t] * keys[t][d] for t in range(L)) for d in range(D_V)]
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)
