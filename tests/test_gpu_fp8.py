"""Decode over the FP8 latent cache on the GPU vs the oracle, through the C ABI.

The oracle decodes the same E4M3 bytes and scales exactly (FP64), so the
gates are the BF16 path's: the kernel's conversion to BF16 is exact, and the
remaining differences are FP32 accumulation, the per-token scale product and
the BF16 rounding of the softmax weights and of the output.
"""

import numpy as np
import pytest

import oracle
from gpu_util import log, score
from workloads import FP8_PAGE_BYTES, make_fp8_cache, make_inputs, make_workload_inputs, pack_fp8_pages

pytestmark = pytest.mark.gpu

# the organisation --decode-kernel forces for the whole run (None: default)
_forced_kernel = None


@pytest.fixture(autouse=True)
def _note_forced_kernel(request):
    global _forced_kernel
    _forced_kernel = request.config.getoption("--decode-kernel")
    yield


def _skip_beyond_16_row_limit(rows):
    """A run forced onto the 16-row organisation cannot decode FP8 query
    blocks above 64 rows (the call returns MLA_ERR_UNSUPPORTED by design)."""
    if _forced_kernel == "rows16" and rows > 64:
        pytest.skip("the forced 16-row FP8 organisation stops at 64 rows")


def _run(inp, codes, rope, scales, num_partitions=0, use_meta=True):
    import torch
    import mla_paged_kv_02_amd as mla
    _skip_beyond_16_row_limit(inp.h_q * inp.s_q)
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    pages = torch.from_numpy(pack_fp8_pages(codes, rope, scales)).cuda()
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(inp.seqlens).cuda()
    meta = mla.get_split_metadata(sl, inp.h_q, inp.s_q, num_partitions, fp8=True) if use_meta else None
    out, lse = mla.decode_fwd_fp8(q, pages, bt, sl, inp.scale, inp.causal, meta=meta,
                                  num_partitions=num_partitions)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def _check(inp, codes, rope, scales, tag, num_partitions=0, seqs=None, use_meta=True):
    log(f"[case] fp8 {tag} B={inp.batch} s_q={inp.s_q} h_q={inp.h_q} causal={inp.causal} parts={num_partitions}")
    out, lse = _run(inp, codes, rope, scales, num_partitions, use_meta)
    ref_out, ref_lse = oracle.mla_decode_fp8_ref(inp.q_bits, codes, rope, scales, inp.block_table, inp.seqlens,
                                                 inp.scale, inp.causal, seqs=seqs)
    s = score(out, lse, ref_out, ref_lse, seqs=seqs)
    log(f"  {s}")
    assert s.ok(), str(s)
    return out, lse


FP8_CASES = [
    # (seqlens, s_q, h_q, causal)
    ([37, 100], 1, 16, False),
    ([1, 63, 64, 65, 127, 128, 129, 300], 1, 16, False),
    ([0, 5, 0, 200], 1, 16, False),
    ([700, 1], 1, 32, False),
    ([130, 257, 64], 1, 64, False),
    ([1, 70, 129], 2, 16, True),
    ([90, 45], 1, 24, False),
    ([150], 3, 8, True),
    ([40, 3, 129], 4, 16, True),
    # 64-row blocks with the FP8 fill: one, two, several per sequence
    ([1, 64, 65, 700], 1, 64, False),
    ([200, 333], 1, 128, False),
    ([2, 3, 65, 190], 2, 128, True),
    ([150, 3, 1000, 64, 0], 8, 128, True),
    ([300, 2, 77], 16, 64, False),
    # 64-row blocks whose last block is partly past M (M = 80, M = 120)
    ([130, 70, 3], 1, 80, False),
    ([1, 200, 65], 3, 40, True),
]


@pytest.mark.parametrize("case", range(len(FP8_CASES)))
def test_fp8_small_shapes(case):
    seqlens, s_q, h_q, causal = FP8_CASES[case]
    inp = make_inputs(seqlens, s_q, h_q, seed=300 + case, causal=causal)
    codes, rope, scales = make_fp8_cache(inp, seed=400 + case)
    _check(inp, codes, rope, scales, f"small[{case}]", use_meta=case % 2 == 0)


@pytest.mark.parametrize("case", [c for c, k in enumerate(FP8_CASES) if k[1] * k[2] <= 64])
def test_fp8_small_shapes_16_row_organisation(case, plan_override):
    """The 16-row FP8 organisation (each wave converts its own key stripe
    into BF16 before both products), which the default plan no longer picks,
    on every small case it supports (up to 64 rows)."""
    plan_override(kernel="rows16")
    seqlens, s_q, h_q, causal = FP8_CASES[case]
    inp = make_inputs(seqlens, s_q, h_q, seed=300 + case, causal=causal)
    codes, rope, scales = make_fp8_cache(inp, seed=400 + case)
    _check(inp, codes, rope, scales, f"small-rows16[{case}]", use_meta=case % 2 == 0)


@pytest.mark.parametrize("parts", [1, 8, 64, 512])
@pytest.mark.parametrize("h_q", [16, 64, 128])
def test_fp8_forced_splits(parts, h_q):
    inp = make_inputs([900, 3, 2049, 64, 1500], 1, h_q, seed=310 + parts)
    codes, rope, scales = make_fp8_cache(inp, seed=410 + parts)
    _check(inp, codes, rope, scales, f"splits h_q={h_q}", num_partitions=parts)


@pytest.mark.parametrize("h_q,kernel", [(16, None), (64, None), (16, "rows16")])
def test_fp8_poisoned_tails_are_ignored(h_q, kernel, plan_override):
    """Unused rows of last pages hold NaN latent bytes, NaN rotary values and
    NaN scales: the output must be bitwise what clean tails give."""
    plan_override(kernel=kernel)
    inp = make_inputs([70, 5, 129, 64], 2, h_q, seed=320, causal=True)
    codes, rope, scales = make_fp8_cache(inp, seed=420)
    out0, lse0 = _check(inp, codes, rope, scales, "clean tails")
    pc, pr, ps = codes.copy(), rope.copy(), scales.copy()
    for b, n in enumerate(inp.seqlens):
        n = int(n)
        if n % 64:
            phys = int(inp.block_table[b, n // 64])
            pc[phys, n % 64:] = 0x7F
            pr[phys, n % 64:] = 0x7FC0
            ps[phys, n % 64:] = np.float32("nan")
    out1, lse1 = _run(inp, pc, pr, ps)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("h_q", [16, 64])
@pytest.mark.parametrize("mode", ["fused", "kernel"])
def test_fp8_combine_modes(mode, h_q, plan_override):
    plan_override(merge=mode)
    inp = make_inputs([0, 900, 3, 2049, 64, 1500, 0, 777], 1, h_q, seed=330)
    codes, rope, scales = make_fp8_cache(inp, seed=430)
    for parts in (8, 64):
        _check(inp, codes, rope, scales, f"combine {mode}", num_partitions=parts)


@pytest.mark.parametrize("h_q,s_q,kernel", [(16, 1, None), (64, 1, None), (128, 2, None), (16, 1, "rows16")])
def test_fp8_reference_restart_on_dominant_key(h_q, s_q, kernel, plan_override):
    """Queries of 1.0 and, late in each sequence, a token whose latent values
    are all 448 * (0.5/448) = 0.5 and whose rotary values are 32: its score
    (512 * 0.5 + 64 * 32 = 2304 before the 1/24 scale, ~1.4e2 in log2 units)
    is far above the others (~1e1) and the first maximum plus the headroom,
    so the kernel must raise the reference and restart the segment. The
    output is then ~0.5, inside the range the absolute output gate is stated
    for (a BF16 output of magnitude 8 alone may round by 0.031), and must
    match the oracle."""
    import dataclasses
    plan_override(kernel=kernel)
    inp = make_inputs([3000, 700, 150], s_q, h_q, seed=340)
    inp = dataclasses.replace(inp, q_bits=np.full_like(inp.q_bits, 0x3F80))
    codes, rope, scales = make_fp8_cache(inp, seed=440)
    for b, t in ((0, 2900), (1, 650), (2, 100)):
        phys, r = inp.block_table[b, t // 64], t % 64
        codes[phys, r] = 0x7E
        scales[phys, r] = np.float32(0.5 / 448.0)
        rope[phys, r] = 0x4200
    for parts in (0, 16):
        out, lse = _check(inp, codes, rope, scales, f"dominant key parts={parts}", num_partitions=parts)
        assert np.all(np.isfinite(lse))


@pytest.mark.parametrize("name", ["memory_bound", "long_context", "compute_leaning", "multi_token"])
def test_fp8_workload_full_size(name):
    inp = make_workload_inputs(name)
    codes, rope, scales = make_fp8_cache(inp, seed=450)
    _check(inp, codes, rope, scales, name, seqs=list(range(inp.batch)))


def test_fp8_rejects_large_query_blocks_on_the_16_row_organisation(plan_override):
    """Forced onto the 16-row FP8 kernel, a 128-row query block is
    refused (that kernel stops at four row blocks)."""
    import torch
    import mla_paged_kv_02_amd as mla
    plan_override(kernel="rows16")
    inp = make_inputs([100], 1, 128, seed=350)
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    pages = torch.zeros((inp.num_pages, FP8_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(inp.seqlens).cuda()
    with pytest.raises(mla.MlaError, match="UNSUPPORTED"):
        mla.decode_fwd_fp8(q, pages, bt, sl, inp.scale, False)


def _append_fp8_case(inp, tag, count=True):
    """Append into an FP8 cache on the GPU; the whole page buffer must equal
    the oracle's pages bit for bit, and the skipped count must match."""
    import torch
    import mla_paged_kv_02_amd as mla
    log(f"[case] fp8 append {tag} B={inp.batch} s_new={inp.s_new} pages={inp.kv_bits.shape[0]}")
    codes, rope, scales = make_fp8_cache(inp, seed=460)
    pages = torch.from_numpy(pack_fp8_pages(codes, rope, scales)).cuda()
    new = torch.from_numpy(np.ascontiguousarray(inp.new_bits).view(np.int16)).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).cuda()
    sl = torch.from_numpy(inp.seqlens).cuda()
    skipped = torch.zeros((), dtype=torch.int32, device="cuda") if count else None
    mla.kv_append_fp8(new, sl, bt, pages, skipped)
    torch.cuda.synchronize()
    rc, rr, rs, rskip = oracle.kv_append_fp8_ref(codes, rope, scales, inp.new_bits, inp.block_table, inp.seqlens)
    got = pages.cpu().numpy()
    want = pack_fp8_pages(rc, rr, rs)
    bad = np.argwhere(np.any(got != want, axis=1))
    assert bad.size == 0, f"{len(bad)} pages differ, first {bad[:4].ravel().tolist()}"
    if count:
        assert int(skipped.item()) == rskip
    return rc, rr, rs


@pytest.mark.parametrize("s_new", [1, 3, 70])
def test_fp8_append_ragged(s_new):
    from workloads import make_append_inputs
    inp = make_append_inputs([0, 1, 5, 63, 64, 65, 130, 333], s_new, seed=470 + s_new, extra_blocks=1)
    _append_fp8_case(inp, f"ragged s_new={s_new}")


def test_fp8_append_holes_and_extremes():
    import oracle_pins as P
    for k, inp in enumerate(P._append_cases(seed=480)):
        nb = inp.new_bits.copy()
        # zero rows, a row with one huge value, tiny and negative-zero values
        nb[0, 0, :512] = 0
        nb[0, 1, :512] = 0x0001
        nb[0, 1, 7] = 0x7F00
        nb[0, 2, :512] = 0x8000
        if nb.shape[1] > 4:
            # rows of only tiny magnitudes: BF16 subnormals (the scale, amax / 448,
            # is then an FP32 subnormal) and the smallest normal binades, both signs
            i = np.arange(512)
            nb[0, 3, :512] = ((i % 127) + 1) | ((i % 3 == 0) << 15)
            nb[0, 4, :512] = ((1 + i % 8) << 7) | (i * 37 % 128) | ((i % 5 == 0) << 15)
        _append_fp8_case(type(inp)(inp.seqlens, inp.block_table, inp.kv_bits, nb), f"holes[{k}]")


def _midpoint_rows(n_rows):
    """BF16 rows whose values put the FP32 quotient fl32(x / scale) exactly on
    an E4M3 midpoint (so that only the exact quotient decides the code): for
    several row maxima, every positive BF16 value x <= amax with that
    property, both signs, after the row maximum itself."""
    from workloads import bf16_round_bits
    grid = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    xs_all = (np.arange(0x0080, 0x7F00, dtype=np.uint32) << 16).view(np.float32)
    rows = []
    for amax in (11.0, 3.0, 5.0, 6.5, 9.0, 13.0, 0.75, 1.5, 1e-20, 3e20):
        amax = float((bf16_round_bits(np.array([amax], dtype=np.float32)).astype(np.uint32) << 16)
                     .view(np.float32)[0])
        s = np.float32(amax) / np.float32(448.0)
        xs = xs_all[xs_all <= amax]
        hit = xs[np.isin((xs / s).astype(np.float32).astype(np.float64), mids)]
        vals = np.concatenate([hit, -hit])
        for k in range(0, max(len(vals), 1), 511):
            row = np.zeros(576, dtype=np.float32)
            row[0] = amax
            chunk = vals[k:k + 511]
            row[1:1 + len(chunk)] = chunk
            rows.append(row)
    rows = np.array(rows[:n_rows], dtype=np.float32)
    bits = bf16_round_bits(rows)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), rows), "rows not exact in BF16"
    return bits


def test_fp8_append_exact_quotient_at_midpoints():
    """Values whose FP32 quotient x / scale lands exactly on an E4M3 midpoint
    (for amax = 11, x = 1.03125 gives 42, between 40 and 44, while the
    exact quotient is just above 42): the codes must be those of the exact
    quotient, bit for bit with the oracle."""
    from workloads import AppendInputs, make_append_inputs
    base = make_append_inputs([64, 130, 200, 17], 8, seed=495)
    rows = _midpoint_rows(base.new_bits.shape[0] * base.new_bits.shape[1])
    nb = base.new_bits.copy().reshape(-1, 576)
    nb[:rows.shape[0]] = rows
    log(f"[case] fp8 append midpoint rows: {rows.shape[0]} rows")
    _append_fp8_case(AppendInputs(base.seqlens, base.block_table, base.kv_bits, nb.reshape(base.new_bits.shape)),
                     "midpoints")


def test_fp8_append_workload_and_decode():
    """The chunked-prefill append into an FP8 cache, then decode of the last
    tokens over it, against the oracle's cache and decode."""
    import torch
    import mla_paged_kv_02_amd as mla
    from workloads import make_append_inputs
    from workloads import AppendInputs
    seqlens = [300, 64, 2, 129, 1000]
    s_q = 4
    dec = make_inputs(seqlens, s_q, 16, seed=491, causal=True)
    new_bits = make_append_inputs(seqlens, s_q, seed=490).new_bits
    inp = AppendInputs(dec.seqlens, dec.block_table, dec.kv_bits, new_bits)
    rc, rr, rs = _append_fp8_case(inp, "then decode")
    _check(dec, rc, rr, rs, "decode after fp8 append")


def test_fp8_append_full_size():
    from workloads import make_append_workload
    inp = make_append_workload("append_prefill_chunk")
    _append_fp8_case(inp, "append_prefill_chunk")


def test_fp8_pages_past_4_gib():
    """FP8 pages at the top of a 4.3 GB page buffer (offsets past 2^32 bytes):
    decode against the oracle on the same logical content."""
    import torch
    inp = make_inputs([300, 70, 129], 1, 16, seed=93)
    codes, rope, scales = make_fp8_cache(inp, seed=94)
    nb = inp.num_pages
    total = 105000                                  # 105000 * 41216 B = 4.3 GB
    shift = total - nb
    log(f"[case] fp8 pages past 4 GiB: {total} pages, used at {shift}..")
    big = torch.empty((total, FP8_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    big[shift:] = torch.from_numpy(pack_fp8_pages(codes, rope, scales)).cuda()
    table = np.where(inp.block_table >= 0, inp.block_table + shift, -1).astype(np.int32)
    import mla_paged_kv_02_amd as mla
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = mla.decode_fwd_fp8(q, big, torch.from_numpy(table).cuda(), torch.from_numpy(inp.seqlens).cuda(),
                                  inp.scale, False)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.mla_decode_fp8_ref(inp.q_bits, codes, rope, scales, inp.block_table, inp.seqlens,
                                                 inp.scale, False)
    s = score(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref_out, ref_lse)
    log(f"  {s}")
    assert s.ok(), str(s)
    del big
    torch.cuda.empty_cache()
