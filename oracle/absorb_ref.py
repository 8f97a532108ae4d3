"""Reference for the weight-absorption steps on either side of MLA decode.

TEST INFRASTRUCTURE ONLY (see the package docstring). No GPU code, no shared
helpers with the HIP library.

Source: page "MLA 和 MHA 的 Kernel 区别" (MLA vs MHA kernel differences),
section "内存布局和 KV Cache 大小" and the MLA decode pseudo-code: keys and
values are up-projections of the cached latent row, K_h = c_KV W_UK_h and
V_h = c_KV W_UV_h, with W_UK_h of shape [512, d_nope] and W_UV_h of shape
[512, d_v] per head h. Folding W_UK_h into the query gives the absorbed query
q_abs_h = W_UK_h q_nope_h (a 512-vector), so the score is
<q_abs_h, c_KV> + <q_rope_h, k_rope>; the latent output o_lat_h (the softmax
average of c_KV rows) becomes the head output o_h = o_lat_h W_UV_h.

Readings: the rotary part of the query passes through unchanged (it meets
the cache's rotary part directly); all arithmetic is float64.
"""

from __future__ import annotations

import numpy as np


def absorb_q_ref(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_nope [T, H, dn], q_rope [T, H, 64], w_uk [H, 512, dn]
    -> q_abs [T, H, 576] = [W_UK_h q_nope ; q_rope] per token and head."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    tokens, heads, _ = q_nope.shape
    out = np.empty((tokens, heads, 512 + q_rope.shape[-1]))
    for h in range(heads):
        out[:, h, :512] = q_nope[:, h, :] @ w_uk[h].T     # [T, dn] x [dn, 512]
    out[:, :, 512:] = np.asarray(q_rope, dtype=np.float64)
    return out


def absorb_o_ref(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o_lat [T, H, 512], w_uv [H, 512, dv] -> o [T, H, dv] = o_lat_h W_UV_h."""
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    tokens, heads, _ = o_lat.shape
    out = np.empty((tokens, heads, w_uv.shape[-1]))
    for h in range(heads):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[h]             # [T, 512] x [512, dv]
    return out
