"""MLA paged decode on MI355X (gfx950): Python binding of libmla_decode.so.

Two calls, as on the FlashMLA overview page (flash_api.cpp walk-through):
the split metadata once per decode step, then the attention call once per
layer.

    meta = get_split_metadata(seqlens, h_q, s_q)
    out, lse = decode_fwd(q, kv_cache, block_table, seqlens, scale, causal, meta=meta)

This module only checks and marshals arguments; every step of the
computation runs in the library's HIP kernels. torch provides device memory
and the current stream.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

from ._lib import MlaError, check, lib  # noqa: F401

HEAD_DIM = 576
HEAD_DIM_V = 512
PAGE_SIZE = 64
FP8_PAGE_BYTES = 41216   # 64 x 512 E4M3 latent + 64 x 64 BF16 rotary + 64 FP32 scales

__all__ = ["SplitMeta", "get_split_metadata", "decode_fwd", "decode_fwd_fp8", "kv_append", "kv_append_fp8", "absorb_q", "absorb_o", "mha_decode_fwd", "split_metadata_host",
           "metadata_bytes", "workspace_bytes", "default_num_partitions", "MlaError"]


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, dtype, device=None, ndim=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def metadata_bytes(batch: int, h_q: int, s_q: int, num_partitions: int = 0) -> int:
    return int(lib().mla_metadata_bytes(batch, h_q, s_q, num_partitions))


def workspace_bytes(batch: int, h_q: int, s_q: int, num_partitions: int = 0) -> int:
    return int(lib().mla_workspace_bytes(batch, h_q, s_q, num_partitions))


def default_num_partitions(h_q: int, s_q: int) -> int:
    return int(lib().mla_default_num_partitions(h_q, s_q))


@dataclasses.dataclass
class SplitMeta:
    """Split-KV plan of one decode step (device buffer plus the arguments it
    was built for). Reuse it for every layer of the step."""

    metadata: torch.Tensor
    batch: int
    h_q: int
    s_q: int
    num_partitions: int
    fp8: bool = False


def get_split_metadata(seqlens: torch.Tensor, h_q: int, s_q: int,
                       num_partitions: int = 0, fp8: bool = False) -> SplitMeta:
    """Build the split plan on the device, on the current stream; ``fp8``
    builds the plan of decode_fwd_fp8 (mla_get_split_metadata_fp8)."""
    _require(seqlens, "seqlens", torch.int32, ndim=1)
    batch = seqlens.shape[0]
    nbytes = metadata_bytes(batch, h_q, s_q, num_partitions)
    if nbytes == 0:
        raise ValueError(f"unsupported shape batch={batch} h_q={h_q} s_q={s_q}")
    meta = torch.empty(nbytes // 4, dtype=torch.int32, device=seqlens.device)
    fn = lib().mla_get_split_metadata_fp8 if fp8 else lib().mla_get_split_metadata
    check(fn(seqlens.data_ptr(), batch, h_q, s_q, num_partitions, meta.data_ptr(), nbytes,
             _stream_ptr(seqlens.device)),
          "mla_get_split_metadata_fp8" if fp8 else "mla_get_split_metadata")
    return SplitMeta(meta, batch, h_q, s_q, num_partitions, fp8)


def split_metadata_host(seqlens, h_q: int, s_q: int, num_partitions: int) -> np.ndarray:
    """The same plan computed on the host (no GPU), as an int32 array."""
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    batch = sl.shape[0]
    nbytes = metadata_bytes(batch, h_q, s_q, num_partitions)
    if nbytes == 0:
        raise ValueError("unsupported shape")
    meta = np.zeros(nbytes // 4, dtype=np.int32)
    check(lib().mla_get_split_metadata_host(sl.ctypes.data, batch, h_q, s_q, num_partitions,
                                            meta.ctypes.data, nbytes),
          "mla_get_split_metadata_host")
    return meta


def decode_fwd(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
               seqlens: torch.Tensor, softmax_scale: float, causal: bool,
               meta: Optional[SplitMeta] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None,
               num_partitions: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLA decode attention for one layer.

    q [B, s_q, h_q, 576] bf16; kv_cache [num_pages, 64, 1, 576] (or
    [num_pages, 64, 576]) bf16; block_table [B, max_blocks] int32;
    seqlens [B] int32. Returns out [B, s_q, h_q, 512] bf16 and
    lse [B, s_q, h_q] float32. Without ``meta`` the call builds the plan
    itself inside its workspace.
    """
    _require(kv_cache, "kv_cache", torch.bfloat16, device=q.device)
    if kv_cache.dim() == 4:
        if tuple(kv_cache.shape[1:]) != (PAGE_SIZE, 1, HEAD_DIM):
            raise ValueError(f"kv_cache must be [num_pages, 64, 1, 576], got {tuple(kv_cache.shape)}")
    elif kv_cache.dim() == 3:
        if tuple(kv_cache.shape[1:]) != (PAGE_SIZE, HEAD_DIM):
            raise ValueError(f"kv_cache must be [num_pages, 64, 576], got {tuple(kv_cache.shape)}")
    else:
        raise ValueError("kv_cache must have 3 or 4 dims")
    if meta is not None and meta.fp8:
        raise ValueError("meta was built for decode_fwd_fp8 (fp8=True)")
    return _decode(lib().mla_decode_fwd, "mla_decode_fwd", q, kv_cache, block_table, seqlens, softmax_scale,
                   causal, meta, out, lse, workspace, num_partitions)


def decode_fwd_fp8(q: torch.Tensor, kv_pages: torch.Tensor, block_table: torch.Tensor,
                   seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                   meta: Optional[SplitMeta] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   num_partitions: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """decode_fwd over an FP8 latent cache (mla_decode_fwd_fp8): kv_pages is
    uint8 [num_pages, 41216] in the page layout of include/mla_decode_fp8.h
    (E4M3 latent rows, BF16 rotary rows, FP32 per-token scales). Query
    blocks of h_q * s_q <= 64 rows."""
    _require(kv_pages, "kv_pages", torch.uint8, device=q.device, ndim=2)
    if kv_pages.shape[1] != FP8_PAGE_BYTES:
        raise ValueError(f"kv_pages must be [num_pages, {FP8_PAGE_BYTES}], got {tuple(kv_pages.shape)}")
    if meta is not None and not meta.fp8:
        raise ValueError("decode_fwd_fp8 needs the plan from get_split_metadata(..., fp8=True)")
    return _decode(lib().mla_decode_fwd_fp8, "mla_decode_fwd_fp8", q, kv_pages, block_table, seqlens,
                   softmax_scale, causal, meta, out, lse, workspace, num_partitions)


def _decode(fn, name, q, kv_cache, block_table, seqlens, softmax_scale, causal, meta, out, lse, workspace,
            num_partitions):
    dev = q.device
    _require(q, "q", torch.bfloat16, ndim=4)
    bsz, s_q, h_q, d = q.shape
    if d != HEAD_DIM:
        raise ValueError(f"q head dim must be {HEAD_DIM}, got {d}")
    _require(block_table, "block_table", torch.int32, device=dev, ndim=2)
    _require(seqlens, "seqlens", torch.int32, device=dev, ndim=1)
    if block_table.shape[0] != bsz or seqlens.shape[0] != bsz:
        raise ValueError("block_table and seqlens must have one row per sequence")
    if meta is not None:
        if (meta.batch, meta.h_q, meta.s_q) != (bsz, h_q, s_q):
            raise ValueError("meta was built for a different batch/h_q/s_q")
        num_partitions = meta.num_partitions
    if out is None:
        out = torch.empty((bsz, s_q, h_q, HEAD_DIM_V), dtype=torch.bfloat16, device=dev)
    else:
        _require(out, "out", torch.bfloat16, device=dev, ndim=4)
        if tuple(out.shape) != (bsz, s_q, h_q, HEAD_DIM_V):
            raise ValueError("out has the wrong shape")
    if lse is None:
        lse = torch.empty((bsz, s_q, h_q), dtype=torch.float32, device=dev)
    else:
        _require(lse, "lse", torch.float32, device=dev, ndim=3)
        if tuple(lse.shape) != (bsz, s_q, h_q):
            raise ValueError("lse has the wrong shape")
    need = workspace_bytes(bsz, h_q, s_q, num_partitions)
    if need == 0:
        raise ValueError(f"unsupported shape B={bsz} h_q={h_q} s_q={s_q}")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous buffer of >= {need} bytes")
    status = fn(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1],
        seqlens.data_ptr(), bsz, s_q, h_q, kv_cache.shape[0], ctypes.c_float(softmax_scale),
        int(bool(causal)), meta.metadata.data_ptr() if meta is not None else None,
        num_partitions, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), lse.data_ptr(), _stream_ptr(dev))
    check(status, name)
    return out, lse


def check_decode_inputs(block_table: torch.Tensor, seqlens: torch.Tensor, num_pages: int,
                        violations: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Count on the device the decode-precondition violations of a block
    table and lengths (mla_check_decode_inputs): lengths outside
    [0, 64 * max_blocks] and table entries the decode would read outside
    [0, num_pages). Returns the int32 scalar tensor the count is written to
    (``violations`` if given), on the stream; 0 means the inputs are valid."""
    dev = block_table.device
    _require(block_table, "block_table", torch.int32, device=dev, ndim=2)
    _require(seqlens, "seqlens", torch.int32, device=dev, ndim=1)
    if block_table.shape[0] != seqlens.shape[0]:
        raise ValueError("block_table and seqlens must have one row per sequence")
    if violations is None:
        violations = torch.empty((), dtype=torch.int32, device=dev)
    else:
        _require(violations, "violations", torch.int32, device=dev)
        if violations.numel() != 1:
            raise ValueError("violations must hold one int32")
    check(lib().mla_check_decode_inputs(block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(),
                                        seqlens.shape[0], int(num_pages), violations.data_ptr(), _stream_ptr(dev)),
          "mla_check_decode_inputs")
    return violations


def kv_append(new_rows: torch.Tensor, seqlens: torch.Tensor, block_table: torch.Tensor,
              kv_cache: torch.Tensor, skipped: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Write the new tokens' cache rows into the paged cache (mla_kv_append).

    new_rows [B, s_new, 576] bf16; seqlens [B] int32 holds the cache lengths
    after the append (token i of sequence b lands at position
    N_b - s_new + i); block_table [B, max_blocks] int32; kv_cache
    [num_pages, 64, 1, 576] (or [num_pages, 64, 576]) bf16, updated in place.
    ``skipped`` (int32 scalar tensor, optional) is incremented for each token
    whose page is missing from the table. Returns kv_cache.
    """
    dev = new_rows.device
    _require(new_rows, "new_rows", torch.bfloat16, ndim=3)
    bsz, s_new, d = new_rows.shape
    if d != HEAD_DIM:
        raise ValueError(f"new_rows head dim must be {HEAD_DIM}, got {d}")
    _require(kv_cache, "kv_cache", torch.bfloat16, device=dev)
    if tuple(kv_cache.shape[1:]) not in ((PAGE_SIZE, 1, HEAD_DIM), (PAGE_SIZE, HEAD_DIM)):
        raise ValueError(f"kv_cache must be [num_pages, 64, 1, 576], got {tuple(kv_cache.shape)}")
    _require(block_table, "block_table", torch.int32, device=dev, ndim=2)
    _require(seqlens, "seqlens", torch.int32, device=dev, ndim=1)
    if block_table.shape[0] != bsz or seqlens.shape[0] != bsz:
        raise ValueError("block_table and seqlens must have one row per sequence")
    if skipped is not None:
        _require(skipped, "skipped", torch.int32, device=dev)
        if skipped.numel() != 1:
            raise ValueError("skipped must hold one int32")
    check(lib().mla_kv_append(new_rows.data_ptr(), bsz, s_new, seqlens.data_ptr(), block_table.data_ptr(),
                              block_table.shape[1], kv_cache.data_ptr(), kv_cache.shape[0],
                              skipped.data_ptr() if skipped is not None else None, _stream_ptr(dev)),
          "mla_kv_append")
    return kv_cache


def kv_append_fp8(new_rows: torch.Tensor, seqlens: torch.Tensor, block_table: torch.Tensor,
                  kv_pages: torch.Tensor, skipped: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kv_append into an FP8 cache (mla_kv_append_fp8): each placed token's
    latent part is quantised to E4M3 with one FP32 scale, its rotary part
    copied. kv_pages uint8 [num_pages, 41216], updated in place. Returns
    kv_pages."""
    dev = new_rows.device
    _require(new_rows, "new_rows", torch.bfloat16, ndim=3)
    bsz, s_new, d = new_rows.shape
    if d != HEAD_DIM:
        raise ValueError(f"new_rows head dim must be {HEAD_DIM}, got {d}")
    _require(kv_pages, "kv_pages", torch.uint8, device=dev, ndim=2)
    if kv_pages.shape[1] != FP8_PAGE_BYTES:
        raise ValueError(f"kv_pages must be [num_pages, {FP8_PAGE_BYTES}], got {tuple(kv_pages.shape)}")
    _require(block_table, "block_table", torch.int32, device=dev, ndim=2)
    _require(seqlens, "seqlens", torch.int32, device=dev, ndim=1)
    if block_table.shape[0] != bsz or seqlens.shape[0] != bsz:
        raise ValueError("block_table and seqlens must have one row per sequence")
    if skipped is not None:
        _require(skipped, "skipped", torch.int32, device=dev)
        if skipped.numel() != 1:
            raise ValueError("skipped must hold one int32")
    check(lib().mla_kv_append_fp8(new_rows.data_ptr(), bsz, s_new, seqlens.data_ptr(), block_table.data_ptr(),
                                  block_table.shape[1], kv_pages.data_ptr(), kv_pages.shape[0],
                                  skipped.data_ptr() if skipped is not None else None, _stream_ptr(dev)),
          "mla_kv_append_fp8")
    return kv_pages


def absorb_q(q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk: torch.Tensor,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Absorbed decode query (mla_absorb_q): [W_UK_h q_nope ; q_rope] per token
    and head. q_nope [..., h, d_nope], q_rope [..., h, 64] bf16 with the same
    leading dims (e.g. [B, s_q]); w_uk [h, 512, d_nope] bf16. Returns
    [..., h, 576] bf16, the q layout decode_fwd takes."""
    dev = q_nope.device
    _require(q_nope, "q_nope", torch.bfloat16)
    _require(q_rope, "q_rope", torch.bfloat16, device=dev)
    _require(w_uk, "w_uk", torch.bfloat16, device=dev, ndim=3)
    if q_nope.dim() < 2 or q_rope.shape[:-1] != q_nope.shape[:-1] or q_rope.shape[-1] != 64:
        raise ValueError("q_rope must be [..., h, 64] with q_nope's leading dims")
    h, d_nope = q_nope.shape[-2], q_nope.shape[-1]
    if tuple(w_uk.shape) != (h, HEAD_DIM_V, d_nope):
        raise ValueError(f"w_uk must be [{h}, 512, {d_nope}], got {tuple(w_uk.shape)}")
    tokens = q_nope.numel() // (h * d_nope)
    shape = (*q_nope.shape[:-1], HEAD_DIM)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    else:
        _require(out, "out", torch.bfloat16, device=dev)
        if tuple(out.shape) != shape:
            raise ValueError("out has the wrong shape")
    check(lib().mla_absorb_q(q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(), tokens, h, d_nope,
                             out.data_ptr(), _stream_ptr(dev)), "mla_absorb_q")
    return out


def absorb_o(o_lat: torch.Tensor, w_uv_t: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Head outputs from the latent decode output (mla_absorb_o): o_lat W_UV_h
    per token and head. o_lat [..., h, 512] bf16 (decode_fwd's out); w_uv_t
    [h, d_v, 512] bf16, W_UV_h transposed per head. Returns [..., h, d_v] bf16."""
    dev = o_lat.device
    _require(o_lat, "o_lat", torch.bfloat16)
    _require(w_uv_t, "w_uv_t", torch.bfloat16, device=dev, ndim=3)
    if o_lat.dim() < 2 or o_lat.shape[-1] != HEAD_DIM_V:
        raise ValueError("o_lat must be [..., h, 512]")
    h = o_lat.shape[-2]
    if w_uv_t.shape[0] != h or w_uv_t.shape[2] != HEAD_DIM_V:
        raise ValueError(f"w_uv_t must be [{h}, d_v, 512], got {tuple(w_uv_t.shape)}")
    d_v = w_uv_t.shape[1]
    tokens = o_lat.numel() // (h * HEAD_DIM_V)
    shape = (*o_lat.shape[:-1], d_v)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    else:
        _require(out, "out", torch.bfloat16, device=dev)
        if tuple(out.shape) != shape:
            raise ValueError("out has the wrong shape")
    check(lib().mla_absorb_o(o_lat.data_ptr(), w_uv_t.data_ptr(), tokens, h, d_v, out.data_ptr(),
                             _stream_ptr(dev)), "mla_absorb_o")
    return out


def mha_decode_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                   seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                   out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged grouped-query MHA decode (mla_mha_decode_fwd), the contrast case.
    q [B, s_q, h_q, 128]; k_cache, v_cache [num_pages, 64, h_kv, 128] bf16;
    (h_q / h_kv) * s_q <= 16. Returns out [B, s_q, h_q, 128] bf16 and
    lse [B, s_q, h_q] float32."""
    dev = q.device
    _require(q, "q", torch.bfloat16, ndim=4)
    bsz, s_q, h_q, d = q.shape
    if d != 128:
        raise ValueError(f"q head dim must be 128, got {d}")
    _require(k_cache, "k_cache", torch.bfloat16, device=dev, ndim=4)
    _require(v_cache, "v_cache", torch.bfloat16, device=dev, ndim=4)
    if k_cache.shape != v_cache.shape or k_cache.shape[1] != PAGE_SIZE or k_cache.shape[3] != 128:
        raise ValueError("k_cache and v_cache must both be [num_pages, 64, h_kv, 128]")
    h_kv = k_cache.shape[2]
    _require(block_table, "block_table", torch.int32, device=dev, ndim=2)
    _require(seqlens, "seqlens", torch.int32, device=dev, ndim=1)
    if block_table.shape[0] != bsz or seqlens.shape[0] != bsz:
        raise ValueError("block_table and seqlens must have one row per sequence")
    if out is None:
        out = torch.empty((bsz, s_q, h_q, 128), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((bsz, s_q, h_q), dtype=torch.float32, device=dev)
    check(lib().mla_mha_decode_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                   block_table.shape[1], seqlens.data_ptr(), bsz, s_q, h_q, h_kv,
                                   k_cache.shape[0], ctypes.c_float(softmax_scale), int(bool(causal)),
                                   out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)), "mla_mha_decode_fwd")
    return out, lse


def set_plan_override(kernel: Optional[str] = None, merge: Optional[str] = None) -> None:
    """Testing hook (mla_set_plan_override): kernel None | "rows16" | "ws" |
    "fw", merge None | "kernel" | "fused"; None restores the default choice.
    Build plans after setting it."""
    k = {None: -1, "rows16": 0, "ws": 1, "fw": 2}[kernel]
    m = {None: -1, "kernel": 0, "fused": 1}[merge]
    check(lib().mla_set_plan_override(k, m), "mla_set_plan_override")


def check_metadata_host(metadata: np.ndarray, batch: int, h_q: int, s_q: int, num_partitions: int,
                        fp8: bool = False) -> bool:
    """Whether a host copy of a plan matches these call arguments
    (mla_check_metadata_host)."""
    meta = np.ascontiguousarray(metadata, dtype=np.int32)
    st = lib().mla_check_metadata_host(meta.ctypes.data, meta.nbytes, batch, h_q, s_q, num_partitions, int(fp8))
    if st == 1:
        return False
    check(st, "mla_check_metadata_host")
    return True


def timing_enable(enable: bool = True) -> None:
    """Record HIP events around the decode and combine kernels of every
    following decode_fwd call (mla_timing_enable)."""
    check(lib().mla_timing_enable(1 if enable else 0), "mla_timing_enable")


def timing_collect() -> Tuple[float, float, int]:
    """(decode kernel ms summed, combine kernel ms summed, calls) over the calls
    recorded since the last collect; synchronise first (mla_timing_collect)."""
    d = ctypes.c_double()
    c = ctypes.c_double()
    n = ctypes.c_int()
    check(lib().mla_timing_collect(ctypes.byref(d), ctypes.byref(c), ctypes.byref(n)),
          "mla_timing_collect")
    return d.value, c.value, n.value
