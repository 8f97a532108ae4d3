"""Reference for appending new tokens' rows to the paged latent cache.

TEST INFRASTRUCTURE ONLY (see the package docstring). No GPU code, no shared
helpers with the HIP library.

Sources (web pages, cited by title and section):

* FlashMLA overview page (nullthought.net, "FlashMLA Overview"): the cache is
  paged in 64-token blocks, and a block table maps a sequence's logical
  block to a physical page.
* "MLA 和 MHA 的 Kernel 区别", section "内存布局和 KV Cache 大小": per token
  the cache keeps only the compressed row (here 512 latent values plus the
  64-value rotary part, 576 BF16).
* "Unlocking GPU Potential: The Impact of FlashAttention and KV Cache
  Optimization in Long-Text Inference": the cache grows with every generated
  token and its management is part of serving.

Reading where the pages are silent: the s_new new tokens of a sequence are
its last s_new tokens, the same reading the decode reference uses for its
causal mask, so new token i of a sequence holding N tokens after the append
sits at position N - s_new + i. Tokens whose position would be negative are
not written. A token whose block-table entry is missing (past the row) or
names no page is not written and is counted. Values are copied bit for bit.
"""

from __future__ import annotations

import numpy as np

PAGE = 64


def kv_append_ref(kv_bits: np.ndarray, new_bits: np.ndarray, block_table: np.ndarray,
                  seqlens: np.ndarray):
    """Returns (cache after the append, count of tokens that had no page).

    kv_bits [num_pages, 64, 1, 576] uint16 (BF16 bits), not modified;
    new_bits [B, s_new, 576] uint16; block_table [B, max_blocks] int32;
    seqlens [B]: lengths after the append.
    """
    kv = np.array(kv_bits, copy=True)
    bsz, s_new, _ = new_bits.shape
    num_pages = kv.shape[0]
    width = block_table.shape[1]
    skipped = 0
    for b in range(bsz):
        n = int(seqlens[b])
        for i in range(s_new):
            pos = n - s_new + i
            if pos < 0:
                continue
            logical = pos // PAGE
            page = int(block_table[b, logical]) if logical < width else -1
            if page < 0 or page >= num_pages:
                skipped += 1
                continue
            kv[page, pos % PAGE, 0, :] = new_bits[b, i, :]
    return kv, skipped
