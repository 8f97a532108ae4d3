"""Seeded generator for paged MLA decode inputs.

Inputs follow the problem statement of the FlashMLA overview page (BF16 query
and cache, a paged cache with 64-token blocks, variable-length sequences) and
the cache-row shape used throughout: 576 values per token, the first 512 being
the compressed latent c_KV and the last 64 the rotary part.

Recipe (fixed so every size and total is reproducible):

1. ``rng = numpy.random.default_rng(seed)``.
2. Sequence lengths are drawn first when the workload asks for random ones.
3. ``NB = sum(ceil(N_b / 64))`` physical pages; ``perm = rng.permutation(NB)``;
   sequence ``b`` takes the next ``ceil(N_b / 64)`` entries of ``perm`` in
   order. The block-table row width is ``max_b ceil(N_b / 64)`` and unused
   entries hold -1.
4. ``q = rng.standard_normal((B, S_q, H_q, 576), float32)`` and
   ``kv = rng.standard_normal((NB, 64, 1, 576), float32)``, both rounded to
   BF16 with round-to-nearest-even on the bit pattern.
5. ``scale = 1/sqrt(576)`` as float32.

Everything here is input preparation only.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 576      # latent (512) + rotary part (64) per cache row
HEAD_DIM_V = 512    # value width: the latent part of the same row
PAGE_SIZE = 64      # tokens per physical page


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic decode workload."""

    name: str
    seed: int
    batch: int
    s_q: int
    h_q: int
    causal: bool
    seqlens_fixed: Optional[tuple] = None       # explicit lengths, or
    seqlens_uniform: Optional[tuple] = None     # (lo, hi) inclusive, drawn
    description: str = ""

    def draw_seqlens(self, rng: np.random.Generator) -> np.ndarray:
        if self.seqlens_fixed is not None:
            return np.asarray(self.seqlens_fixed, dtype=np.int32)
        lo, hi = self.seqlens_uniform
        return rng.integers(lo, hi, size=self.batch, endpoint=True).astype(np.int32)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, 2, 1, 16, False, seqlens_fixed=(37, 100),
        description="batch 2, seqlens {37,100}, s_q=1, h_q=16"),
    "memory_bound": Workload(
        "memory_bound", 2, 64, 1, 16, False, seqlens_uniform=(3072, 5120),
        description="batch 64, seqlens U[3072,5120], s_q=1, h_q=16"),
    "compute_leaning": Workload(
        "compute_leaning", 3, 128, 1, 128, False, seqlens_fixed=(4096,) * 128,
        description="batch 128, seqlen 4096, s_q=1, h_q=128"),
    "long_context": Workload(
        "long_context", 4, 4, 1, 64, False, seqlens_fixed=(1024, 16384, 32768, 65536),
        description="batch 4, seqlens {1K,16K,32K,64K}, s_q=1, h_q=64"),
    "multi_token": Workload(
        "multi_token", 5, 132, 2, 128, True, seqlens_uniform=(1, 8192),
        description="batch 132, seqlens U[1,8192], s_q=2 causal, h_q=128"),
}


@dataclasses.dataclass
class MlaInputs:
    """Host-side inputs. BF16 tensors are held as their uint16 bit patterns."""

    seqlens: np.ndarray        # int32 [B]
    block_table: np.ndarray    # int32 [B, max_blocks]
    q_bits: np.ndarray         # uint16 [B, S_q, H_q, 576]
    kv_bits: np.ndarray        # uint16 [NB, 64, 1, 576]
    scale: float               # exactly representable in float32
    causal: bool

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q_bits.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q_bits.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.kv_bits.shape[0])


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit pattern (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit pattern -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _standard_normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 25) -> np.ndarray:
    """Draw N(0,1) float32 in one stream and round to BF16 bits, chunk by chunk
    (same values as one big draw, bounded temporary memory)."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    done = 0
    while done < total:
        n = min(chunk, total - done)
        out[done:done + n] = bf16_round_bits(rng.standard_normal(n, dtype=np.float32))
        done += n
    return out.reshape(shape)


def make_inputs(seqlens: Sequence[int], s_q: int, h_q: int, seed: int,
                causal: bool = False, rng: Optional[np.random.Generator] = None,
                extra_blocks: int = 0) -> MlaInputs:
    """Build inputs for explicit sequence lengths.

    ``rng`` lets a workload draw its lengths from the same stream first.
    ``extra_blocks`` widens the block table beyond the longest sequence (the
    extra entries are padding, -1).
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    if seqlens.ndim != 1 or seqlens.size == 0 or (seqlens < 0).any():
        raise ValueError("seqlens must be a non-empty 1-D array of non-negative ints")
    pages = (seqlens.astype(np.int64) + PAGE_SIZE - 1) // PAGE_SIZE
    nb = int(pages.sum())
    perm = rng.permutation(nb).astype(np.int32) if nb > 0 else np.zeros(0, np.int32)
    width = max(int(pages.max()), 1) + int(extra_blocks)
    table = np.full((seqlens.size, width), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[cur:cur + n]
        cur += int(n)
    q_bits = _standard_normal_bf16(rng, (seqlens.size, s_q, h_q, HEAD_DIM))
    kv_bits = _standard_normal_bf16(rng, (max(nb, 1), PAGE_SIZE, 1, HEAD_DIM))
    scale = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))
    return MlaInputs(seqlens, table, q_bits, kv_bits, scale, bool(causal))


def make_workload_inputs(name: str) -> MlaInputs:
    """Inputs of a named workload, with its own seed."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    seqlens = w.draw_seqlens(rng)
    return make_inputs(seqlens, w.s_q, w.h_q, w.seed, w.causal, rng=rng)


def permute_pages(inp: MlaInputs, seed: int) -> MlaInputs:
    """Move every physical page to a new slot and rewrite the block table to
    match. The logical content of every sequence is unchanged."""
    rng = np.random.default_rng(seed)
    nb = inp.num_pages
    pi = rng.permutation(nb).astype(np.int32)
    kv = np.empty_like(inp.kv_bits)
    kv[pi] = inp.kv_bits
    table = inp.block_table.copy()
    valid = table >= 0
    valid &= table < nb
    table[valid] = pi[table[valid]]
    return dataclasses.replace(inp, block_table=table, kv_bits=kv)


def poison_page_tails(inp: MlaInputs, bits: int = 0x7FC0) -> MlaInputs:
    """Fill the unused rows of every partially filled last page with ``bits``
    (a BF16 NaN by default)."""
    kv = inp.kv_bits.copy()
    for b, n in enumerate(inp.seqlens):
        n = int(n)
        if n % PAGE_SIZE == 0:
            continue
        phys = int(inp.block_table[b, n // PAGE_SIZE])
        kv[phys, n % PAGE_SIZE:] = np.uint16(bits)
    return dataclasses.replace(inp, kv_bits=kv)


def poison_block_table_padding(inp: MlaInputs) -> MlaInputs:
    """Fill block-table entries past each sequence's last page with -1 and
    INT32_MAX, alternating."""
    table = inp.block_table.copy()
    for b, n in enumerate(inp.seqlens):
        used = (int(n) + PAGE_SIZE - 1) // PAGE_SIZE
        pad = table.shape[1] - used
        if pad > 0:
            vals = np.where(np.arange(pad) % 2 == 0, -1, np.iinfo(np.int32).max)
            table[b, used:] = vals.astype(np.int32)
    return dataclasses.replace(inp, block_table=table)


@dataclasses.dataclass
class AppendInputs:
    """Host-side inputs of a cache append. BF16 tensors as uint16 bits."""

    seqlens: np.ndarray        # int32 [B], lengths after the append
    block_table: np.ndarray    # int32 [B, max_blocks]
    kv_bits: np.ndarray        # uint16 [NB, 64, 1, 576], the cache before the append
    new_bits: np.ndarray       # uint16 [B, s_new, 576]

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def s_new(self) -> int:
        return int(self.new_bits.shape[1])


def make_append_inputs(seqlens: Sequence[int], s_new: int, seed: int,
                       extra_blocks: int = 0) -> AppendInputs:
    """Pages, block table and prior cache content as for decode (steps 1-4 of
    the recipe, with one query head and token), then the new rows
    ``rng.standard_normal((B, s_new, 576))`` rounded to BF16 from the same
    stream."""
    rng = np.random.default_rng(seed)
    base = make_inputs(seqlens, 1, 1, seed, rng=rng, extra_blocks=extra_blocks)
    new_bits = _standard_normal_bf16(rng, (base.batch, s_new, HEAD_DIM))
    return AppendInputs(base.seqlens, base.block_table, base.kv_bits, new_bits)


# Append workloads: the rows of one decode step of the memory-bound workload,
# and one chunk of chunked prefill (2048 new tokens for each of 32 sequences
# that end up 2048..8192 tokens long).
APPEND_WORKLOADS = {
    "append_decode_step": dict(s_new=1, seed=21, lengths=("uniform", 64, 3072, 5120)),
    "append_prefill_chunk": dict(s_new=2048, seed=22, lengths=("uniform", 32, 2048, 8192)),
}


def make_append_workload(name: str) -> AppendInputs:
    w = APPEND_WORKLOADS[name]
    rng = np.random.default_rng(w["seed"])
    _, n, lo, hi = w["lengths"]
    seqlens = rng.integers(lo, hi, size=n, endpoint=True).astype(np.int32)
    base = make_inputs(seqlens, 1, 1, w["seed"], rng=rng)
    new_bits = _standard_normal_bf16(rng, (n, w["s_new"], HEAD_DIM))
    return AppendInputs(base.seqlens, base.block_table, base.kv_bits, new_bits)


# Absorption workloads: the query and output projections around one decode
# step of the 128-head workloads (d_nope = d_v = 128, as in the 128-head MLA
# models these shapes come from). Weights are N(0, 1/K) so outputs keep unit
# scale.
ABSORB_WORKLOADS = {
    "absorb_compute_leaning": dict(tokens=128, heads=128, d_nope=128, d_v=128, seed=23),
    "absorb_multi_token": dict(tokens=264, heads=128, d_nope=128, d_v=128, seed=24),
}


@dataclasses.dataclass
class AbsorbInputs:
    q_nope: np.ndarray     # uint16 [T, H, d_nope]
    q_rope: np.ndarray     # uint16 [T, H, 64]
    w_uk: np.ndarray       # uint16 [H, 512, d_nope]
    o_lat: np.ndarray      # uint16 [T, H, 512]
    w_uv: np.ndarray       # uint16 [H, 512, d_v]


def make_absorb_inputs(tokens: int, heads: int, d_nope: int, d_v: int, seed: int) -> AbsorbInputs:
    rng = np.random.default_rng(seed)

    def draw(shape, std=1.0):
        return bf16_round_bits((rng.standard_normal(shape, dtype=np.float32) * np.float32(std)))

    q_nope = draw((tokens, heads, d_nope))
    q_rope = draw((tokens, heads, 64))
    w_uk = draw((heads, 512, d_nope), 1.0 / math.sqrt(d_nope))
    o_lat = draw((tokens, heads, 512))
    w_uv = draw((heads, 512, d_v), 1.0 / math.sqrt(512))
    return AbsorbInputs(q_nope, q_rope, w_uk, o_lat, w_uv)


def make_absorb_workload(name: str) -> AbsorbInputs:
    w = ABSORB_WORKLOADS[name]
    return make_absorb_inputs(w["tokens"], w["heads"], w["d_nope"], w["d_v"], w["seed"])


# FP8 latent caches (E4M3 latent bytes, BF16 rotary part, FP32 per-token
# scales; page layout of include/mla_decode_fp8.h).
FP8_PAGE_BYTES = 41216


def _e4m3_grid():
    """Finite non-negative E4M3 values and their codes, from the bit layout
    (bias 7, 3 mantissa bits; exponent field 0 subnormal). Input drawing only."""
    codes = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E (0x7F is NaN)
    exp, man = codes >> 3, codes & 7
    vals = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1 + man / 8.0) * 2.0 ** (exp - 7))
    return vals, codes.astype(np.uint8)


def make_fp8_cache(inp: MlaInputs, seed: int):
    """An FP8 cache for the pages of `inp`: latent bytes whose values are
    about N(0,1) * 112 on the E4M3 grid (nearest grid point, drawn from
    ``default_rng(seed)``), scales U[0.8, 1.2] * 4/448 so the latent values
    are about N(0,1) like the BF16 workloads', each token at its own scale,
    and the rotary part taken from inp's BF16 rows.
    Returns (codes uint8 [P, 64, 512], rope uint16 [P, 64, 64],
    scales float32 [P, 64])."""
    rng = np.random.default_rng(seed)
    pages = inp.kv_bits.shape[0]
    y = rng.standard_normal((pages, PAGE_SIZE, 512), dtype=np.float32) * np.float32(112.0)
    vals, codes = _e4m3_grid()
    mag = np.minimum(np.abs(y), 448.0)
    idx = np.clip(np.searchsorted(vals, mag), 1, vals.size - 1)
    near = np.where(mag - vals[idx - 1] <= vals[idx] - mag, idx - 1, idx)
    lat = codes[near] | np.where(y < 0, 0x80, 0).astype(np.uint8)
    scales = (rng.uniform(0.8, 1.2, size=(pages, PAGE_SIZE)) * (4.0 / 448.0)).astype(np.float32)
    rope = np.ascontiguousarray(inp.kv_bits[:, :, 0, HEAD_DIM_V:])
    return lat.astype(np.uint8), rope, scales


def pack_fp8_pages(codes: np.ndarray, rope: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [P,64,512] u8, rope [P,64,64] u16, scales [P,64] f32) -> the
    device page layout, uint8 [P, 41216]: four groups of 16 tokens, 10,304
    bytes each, holding the group's latent rows, rotary rows, scales."""
    pages = codes.shape[0]
    g = np.empty((pages, 4, 10304), dtype=np.uint8)
    g[:, :, :8192] = codes.reshape(pages, 4, 8192)
    g[:, :, 8192:10240] = np.ascontiguousarray(rope, dtype=np.uint16).view(np.uint8).reshape(pages, 4, 2048)
    g[:, :, 10240:] = np.ascontiguousarray(scales, dtype=np.float32).view(np.uint8).reshape(pages, 4, 64)
    return g.reshape(pages, FP8_PAGE_BYTES)


# Paged multi-head (grouped-query) attention inputs, the contrast case:
# keys and values [num_pages][64][H_kv][D] each, drawn like the MLA cache.
@dataclasses.dataclass
class MhaInputs:
    seqlens: np.ndarray        # int32 [B]
    block_table: np.ndarray    # int32 [B, max_blocks]
    q_bits: np.ndarray         # uint16 [B, S_q, H_q, D]
    k_bits: np.ndarray         # uint16 [NB, 64, H_kv, D]
    v_bits: np.ndarray         # uint16 [NB, 64, H_kv, D]
    scale: float
    causal: bool

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])


def make_mha_inputs(seqlens: Sequence[int], s_q: int, h_q: int, h_kv: int, d: int, seed: int,
                    causal: bool = False, rng: Optional[np.random.Generator] = None) -> MhaInputs:
    """Steps 1-3 of the recipe for lengths, pages and table; then q, K and V
    N(0,1) rounded to BF16 from the same stream; scale 1/sqrt(D)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    base = make_inputs(seqlens, 1, 1, seed, rng=rng)
    nb = base.kv_bits.shape[0]
    q = _standard_normal_bf16(rng, (base.batch, s_q, h_q, d))
    k = _standard_normal_bf16(rng, (nb, PAGE_SIZE, h_kv, d))
    v = _standard_normal_bf16(rng, (nb, PAGE_SIZE, h_kv, d))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    return MhaInputs(base.seqlens, base.block_table, q, k, v, scale, bool(causal))


# The contrast workload: the memory-bound decode step under grouped-query
# MHA with 8 KV heads of 128 values, the layout an MHA model of this size
# would cache. Same seed and draw order as the memory-bound workload, so the
# 64 sequence lengths (U[3072, 5120]) are exactly its lengths.
MHA_WORKLOADS = {
    "mha_memory_bound": dict(seed=2, batch=64, lengths=(3072, 5120), s_q=1, h_q=16, h_kv=8, d=128),
}


def make_mha_workload(name: str) -> MhaInputs:
    w = MHA_WORKLOADS[name]
    rng = np.random.default_rng(w["seed"])
    seqlens = rng.integers(w["lengths"][0], w["lengths"][1], size=w["batch"], endpoint=True).astype(np.int32)
    return make_mha_inputs(seqlens, w["s_q"], w["h_q"], w["h_kv"], w["d"], w["seed"], rng=rng)
