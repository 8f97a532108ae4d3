"""Reference for paged multi-head (grouped-query) attention decode, the
contrast case to MLA.

TEST INFRASTRUCTURE ONLY (see the package docstring). No GPU code, no shared
helpers with the HIP library.

Source: page "MLA 和 MHA 的 Kernel 区别" (MLA vs MHA kernel differences),
sections "内存布局和 KV Cache 大小" and "Decode 阶段的 HBM 访问模式" / "MHA
Decode": standard attention keeps a key and a value vector per KV head and
token, and decode reads both for every cached token; each query head scores
the keys of its KV head, takes the softmax and sums that head's values.

Readings: H_q query heads share H_kv KV heads in consecutive groups (query
head h uses KV head h // (H_q / H_kv)); the cache is paged like the MLA one
(64-token pages through a block table) with layout
[num_pages][64][H_kv][D] for keys and for values; the causal rule for
s_q > 1 and the empty-row rule are those of the MLA reference.
"""

from __future__ import annotations

import math

import numpy as np

PAGE = 64


def _bits_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def mha_decode_ref(q_bits, k_bits, v_bits, block_table, seqlens, scale, causal):
    """q_bits [B, s_q, H_q, D], k_bits / v_bits [P, 64, H_kv, D] (BF16 bits).
    Returns out [B, s_q, H_q, D] float64 and lse [B, s_q, H_q] (natural log,
    -inf for a row with no visible key, whose output is zero)."""
    q = _bits_f64(q_bits)
    bsz, s_q, h_q, d = q.shape
    h_kv = k_bits.shape[2]
    group = h_q // h_kv
    scale = float(np.float32(scale))
    out = np.zeros((bsz, s_q, h_q, d))
    lse = np.full((bsz, s_q, h_q), -np.inf)
    for b in range(bsz):
        n = int(seqlens[b])
        if n == 0:
            continue
        t = np.arange(n)
        pages = np.asarray(block_table[b])[t // PAGE]
        k = _bits_f64(k_bits[pages, t % PAGE])          # [n, H_kv, D]
        v = _bits_f64(v_bits[pages, t % PAGE])
        for i in range(s_q):
            L = max(0, min(n, n - s_q + i + 1)) if causal else n
            if L == 0:
                continue
            for h in range(h_q):
                kv = h // group
                s = scale * (k[:L, kv, :] @ q[b, i, h])
                m = s.max()
                e = np.exp(s - m)
                tot = e.sum()
                lse[b, i, h] = m + math.log(tot)
                out[b, i, h] = (e / tot) @ v[:L, kv, :]
    return out, lse


def mha_decode_bruteforce(q, k, v, block_table, seqlens, scale, causal):
    """The same in pure Python with math.fsum, for tiny float64 inputs
    (q [B][s_q][H_q][D], k, v [P][64][H_kv][D])."""
    bsz, s_q, h_q, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    h_kv = len(k[0][0])
    group = h_q // h_kv
    out = [[[[0.0] * d for _ in range(h_q)] for _ in range(s_q)] for _ in range(bsz)]
    lse = [[[-math.inf] * h_q for _ in range(s_q)] for _ in range(bsz)]
    for b in range(bsz):
        n = int(seqlens[b])
        for i in range(s_q):
            L = max(0, min(n, n - s_q + i + 1)) if causal else n
            for h in range(h_q):
                if L == 0:
                    continue
                kv = h // group
                keys = [k[int(block_table[b][t // PAGE])][t % PAGE][kv] for t in range(L)]
                vals = [v[int(block_table[b][t // PAGE])][t % PAGE][kv] for t in range(L)]
                s = [scale * math.fsum(float(q[b][i][h][x]) * float(keys[t][x]) for x in range(d)) for t in range(L)]
                m = max(s)
                ll = m + math.log(math.fsum(math.exp(x - m) for x in s))
                lse[b][i][h] = ll
                p = [math.exp(x - ll) for x in s]
                out[b][i][h] = [math.fsum(p[t] * float(vals[t][x]) for t in range(L)) for x in range(d)]
    return np.array(out), np.array(lse)
