"""HIP path vs the FP64 oracle, element by element, through the C ABI.

Small cases span several pages, ragged tails, empty sequences, the causal
mask and forced splits; the named workloads run at full size, in the launch
configuration the benchmark times, and every sequence of every one is
compared with the oracle (the oracle converts only the pages a sequence
uses, one sequence at a time).
"""

import numpy as np
import pytest

import oracle
from gpu_util import bf16_bits_to_f64, log, run_decode, score
from workloads import (WORKLOADS, make_inputs, make_workload_inputs, permute_pages,
                       poison_block_table_padding, poison_page_tails)

pytestmark = pytest.mark.gpu


def _check(inp, num_partitions=0, seqs=None, use_meta=True, tag=""):
    log(f"[case] {tag} B={inp.batch} s_q={inp.s_q} h_q={inp.h_q} causal={inp.causal} "
        f"lens={inp.seqlens.tolist()[:8]} parts={num_partitions}")
    out, lse = run_decode(inp, num_partitions=num_partitions, use_meta=use_meta)
    ref_out, ref_lse = oracle.mla_decode_ref(inp.q_bits, inp.kv_bits, inp.block_table,
                                             inp.seqlens, inp.scale, inp.causal, seqs=seqs)
    sc = score(out, lse, ref_out, ref_lse, seqs=seqs)
    log(f"       {sc}")
    assert sc.ok(), f"{tag}: {sc}"
    return out, lse


SMALL_CASES = [
    # (seqlens, s_q, h_q, causal)
    ([37, 100], 1, 16, False),
    ([1, 63, 64, 65, 127, 128, 129, 300], 1, 16, False),
    ([0, 5, 0, 200], 1, 16, False),
    ([700, 1], 1, 32, False),
    ([130, 257, 64], 1, 64, False),
    ([200, 333], 1, 128, False),
    ([2, 3, 65, 190], 2, 128, True),
    ([1, 70, 129], 2, 64, True),
    ([90, 45], 1, 24, False),          # rows not a multiple of 16
    ([150], 3, 8, True),               # M = 24, three causal tokens
    ([1000, 17], 1, 16, True),         # causal with s_q = 1 is a no-op
    # larger S_q (speculative / chunked decode), up to the row limit M = 1024
    ([150, 3, 1000, 64], 8, 128, True),
    ([500, 20, 64, 0], 64, 16, True),
    ([300, 2, 77], 16, 64, False),
    ([40, 129], 32, 8, True),
    # 64-row blocks whose last block is partly past M (M = 80, M = 120)
    ([130, 70, 3], 1, 80, False),
    ([200, 64], 3, 40, True),
]


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_small_shapes(case):
    seqlens, s_q, h_q, causal = SMALL_CASES[case]
    inp = make_inputs(seqlens, s_q, h_q, seed=100 + case, causal=causal)
    _check(inp, tag=f"small[{case}]")


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_small_shapes_fused_wave_forced(case, plan_override):
    """Every small case on the 128-row fused-wave organisation: rows past M
    inside its block (down to 8 of 128 in use), ragged tails, empty
    sequences, causal masks, several row blocks per sequence."""
    plan_override(kernel="fw")
    seqlens, s_q, h_q, causal = SMALL_CASES[case]
    inp = make_inputs(seqlens, s_q, h_q, seed=100 + case, causal=causal)
    _check(inp, tag=f"small-fw[{case}]")


@pytest.mark.parametrize("h_q,parts", [(16, 8), (16, 16), (16, 24), (64, 8)])
def test_combine_grid_over_partition_boundaries(h_q, parts, plan_override):
    """More sequences than partition boundaries, merged by the combine
    kernel: its grid follows the boundaries (each split sequence merged once,
    by the group of its first cut) and a tail of blocks writes the empty
    sequences, here five of 37."""
    plan_override(merge="kernel")
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 700, size=37)]
    for e in (0, 5, 17, 30, 36):
        lens[e] = 0
    inp = make_inputs(lens, 1, h_q, seed=50 + parts)
    _check(inp, num_partitions=parts, tag=f"boundary combine h_q={h_q} parts={parts}")


@pytest.mark.parametrize("parts", [1, 8, 24, 64, 512])
@pytest.mark.parametrize("shape", [(16, 1, False), (64, 1, False), (128, 2, True)])
def test_forced_splits(parts, shape):
    h_q, s_q, causal = shape
    inp = make_inputs([900, 3, 2049, 64, 1500], s_q, h_q, seed=7 + parts, causal=causal)
    _check(inp, num_partitions=parts, tag=f"splits h_q={h_q}")


def test_metadata_computed_inside_decode():
    inp = make_inputs([400, 90, 1200], 1, 16, seed=21)
    a = run_decode(inp, num_partitions=64, use_meta=True)
    b = run_decode(inp, num_partitions=64, use_meta=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_poisoned_tails_and_padding_are_ignored():
    inp = make_inputs([37, 100, 129, 1], 2, 16, seed=22, causal=True, extra_blocks=3)
    base = run_decode(inp, num_partitions=16)
    bad = poison_block_table_padding(poison_page_tails(inp))
    got = run_decode(bad, num_partitions=16)
    assert np.array_equal(base[0], got[0]) and np.array_equal(base[1], got[1])


def test_page_permutation_bitwise():
    inp = make_inputs([513, 64, 1000], 1, 64, seed=23)
    a = run_decode(inp, num_partitions=32)
    b = run_decode(permute_pages(inp, 5), num_partitions=32)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_single_token_returns_value_row():
    inp = make_inputs([1, 1, 1], 1, 16, seed=24)
    out, lse = run_decode(inp)
    for b in range(3):
        row = inp.kv_bits[inp.block_table[b, 0], 0, 0, :512]
        assert np.array_equal(out[b, 0], np.broadcast_to(row, (16, 512))), "out != V_0 bitwise"
    _check(inp, tag="single token")


def test_equal_scores_give_mean_of_values():
    inp = make_inputs([300], 1, 16, seed=25)
    inp.q_bits[...] = 0                                   # all scores 0
    out, lse = run_decode(inp)
    assert np.allclose(lse, np.log(300), atol=1e-3)
    _check(inp, tag="equal scores")


def test_empty_sequence_outputs_zero_and_neg_inf():
    inp = make_inputs([0, 10, 0], 2, 16, seed=26, causal=True)
    out, lse = run_decode(inp)
    assert not np.any(out[0]) and not np.any(out[2])
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    _check(inp, tag="empty")


def test_device_metadata_matches_host():
    import torch
    import mla_paged_kv_02_amd as mla
    rng = np.random.default_rng(27)
    for h_q, s_q, parts in [(16, 1, 0), (64, 1, 256), (128, 2, 100), (16, 1, 3000)]:
        seqlens = rng.integers(0, 9000, size=1500).astype(np.int32)
        meta = mla.get_split_metadata(torch.from_numpy(seqlens).cuda(), h_q, s_q, parts)
        host_parts = parts if parts > 0 else mla.default_num_partitions(h_q, s_q)
        host = mla.split_metadata_host(seqlens, h_q, s_q, host_parts)
        dev = meta.metadata.cpu().numpy()
        # the buffer is sized for either decode's plan; compare this plan's
        # ints: header, 8 per partition, 4 per sequence, R counters per sequence
        used = 16 + 8 * int(host[2]) + 4 * int(host[1]) + int(host[8]) * int(host[1])
        assert np.array_equal(dev[:used], host[:used]), f"device metadata differs for h_q={h_q} parts={parts}"
    # more sequences than the scheduler keeps in LDS, and cost lines long
    # enough that partition arithmetic needs more than 32 bits
    for batch, top, parts in [(9000, 3000, 4096), (64, 1 << 24, 60000), (3, 1 << 26, 65536)]:
        seqlens = rng.integers(0, top, size=batch).astype(np.int32)
        meta = mla.get_split_metadata(torch.from_numpy(seqlens).cuda(), 16, 1, parts)
        host = mla.split_metadata_host(seqlens, 16, 1, parts)
        assert np.array_equal(meta.metadata.cpu().numpy(), host), f"device metadata differs, batch={batch}"


@pytest.mark.parametrize("batch", [1, 2, 4, 5, 16, 17, 64, 65, 256, 257, 1024, 1025, 4096, 4097, 8192])
def test_device_metadata_matches_host_at_search_depths(batch):
    """Device plan = host plan at every batch size where the device's search
    of the cost-line starts in LDS changes depth (radix 4: 1, 4, 16, ...
    sequences per probe step) up to the largest batch it keeps in LDS, with a
    quarter of the sequences empty (equal starts) and partition counts below,
    at and above the number of pages."""
    import torch
    import mla_paged_kv_02_amd as mla
    rng = np.random.default_rng(1000 + batch)
    seqlens = rng.integers(1, 3000, size=batch).astype(np.int32)
    seqlens[rng.random(batch) < 0.25] = 0
    if not seqlens.any():
        seqlens[-1] = 65
    pages = int(((seqlens.astype(np.int64) + 63) // 64).sum())
    for parts in sorted({1, 7, 256, min(max(1, pages // 2), 65536), min(pages + 5, 65536)}):
        meta = mla.get_split_metadata(torch.from_numpy(seqlens).cuda(), 16, 1, parts)
        host = mla.split_metadata_host(seqlens, 16, 1, parts)
        dev = meta.metadata.cpu().numpy()
        used = 16 + 8 * int(host[2]) + 4 * int(host[1]) + int(host[8]) * int(host[1])
        assert np.array_equal(dev[:used], host[:used]), f"device metadata differs, batch={batch} parts={parts}"


def test_run_to_run_bitwise():
    inp = make_inputs([3000, 77, 4097], 2, 128, seed=28, causal=True)
    a = run_decode(inp)
    b = run_decode(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_named_workload_full_size(name):
    inp = make_workload_inputs(name)
    _check(inp, seqs=list(range(inp.batch)), tag=f"workload {name}")


def _perturb_other_sequences(inp, keep, seed):
    """New query rows for every sequence not in `keep`, and new cache rows in
    every page that only those sequences use (lengths and the block table
    unchanged, so the split plan is unchanged too)."""
    import dataclasses
    rng = np.random.default_rng(seed)
    q = inp.q_bits.copy()
    kv = inp.kv_bits.copy()
    kept_pages = set()
    for b in keep:
        kept_pages.update(int(x) for x in inp.block_table[b, :(int(inp.seqlens[b]) + 63) // 64])
    others = [b for b in range(inp.batch) if b not in keep]
    for b in others:
        q[b] = rng.integers(0, 1 << 16, size=q[b].shape, dtype=np.uint16) & 0xBFFF   # finite BF16, |x| < 2
        for pg in inp.block_table[b, :(int(inp.seqlens[b]) + 63) // 64]:
            if int(pg) not in kept_pages:
                kv[int(pg)] = (rng.integers(0, 1 << 16, size=kv[int(pg)].shape, dtype=np.uint16) & 0xBFFF)
    return dataclasses.replace(inp, q_bits=q, kv_bits=kv)


@pytest.mark.parametrize("name", ["memory_bound", "long_context", "multi_token"])
def test_batch_independence_full_size(name):
    """Pin (h), batch independence: with the lengths fixed (so the same split
    plan), changing every other sequence's query and cache rows leaves the
    kept sequences' outputs and lse bitwise unchanged. Kept: the shortest,
    the longest and the middle sequence by length (with the default plan the
    longest is split across partitions)."""
    inp = make_workload_inputs(name)
    order = np.argsort(inp.seqlens, kind="stable")
    keep = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2])})
    log(f"[case] batch independence {name}: keep {keep} of {inp.batch}")
    base = run_decode(inp)
    other = run_decode(_perturb_other_sequences(inp, keep, seed=7))
    for b in keep:
        assert np.array_equal(base[0][b], other[0][b]), f"sequence {b} output changed"
        assert np.array_equal(base[1][b], other[1][b]), f"sequence {b} lse changed"
    changed = [b for b in range(inp.batch) if b not in keep and not np.array_equal(base[0][b], other[0][b])]
    assert len(changed) == inp.batch - len(keep), "the perturbation did not reach every other sequence"


@pytest.mark.parametrize("h_q,s_q,causal", [(16, 1, False), (128, 2, True)])
def test_fused_combine_counters_and_modes(h_q, s_q, causal, plan_override):
    """The merge inside the decode kernel (last workgroup of a split
    sequence) against the combine kernel: same results, and the partial
    counters in the metadata are zero again after every call, so repeated
    calls with one metadata buffer agree."""
    import torch
    import mla_paged_kv_02_amd as mla
    from gpu_util import to_device
    inp = make_inputs([0, 900, 3, 2049, 64, 1500, 0, 777], s_q, h_q, seed=31, causal=causal)
    q, kv, bt, sl = to_device(inp)
    ref_out, ref_lse = oracle.mla_decode_ref(inp.q_bits, inp.kv_bits, inp.block_table,
                                             inp.seqlens, inp.scale, inp.causal)
    for parts in (8, 24):
        meta = mla.get_split_metadata(sl, h_q, s_q, parts)
        host = mla.split_metadata_host(inp.seqlens, h_q, s_q, parts)
        results = {}
        for mode in ("fused", "kernel", "fused"):
            plan_override(merge=mode)
            out, lse = mla.decode_fwd(q, kv, bt, sl, inp.scale, inp.causal, meta=meta,
                                      num_partitions=parts)
            torch.cuda.synchronize()
            bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
            lse_h = lse.cpu().numpy()
            sc = score(bits, lse_h, ref_out, ref_lse)
            log(f"[case] fused-combine h_q={h_q} parts={parts} mode={mode}: {sc}")
            assert sc.ok(), f"{mode} parts={parts}: {sc}"
            # the counters (and all of the plan) are as the metadata call wrote
            # them; the buffer is sized for the larger of the BF16 and FP8
            # plans, so only the plan's own ints are compared
            used = 16 + 8 * int(host[2]) + 4 * int(host[1]) + int(host[8]) * int(host[1])
            assert np.array_equal(meta.metadata.cpu().numpy()[:used], host[:used]), f"metadata changed ({mode})"
            if mode in results:
                assert np.array_equal(results[mode][0], bits) and np.array_equal(results[mode][1], lse_h)
            results[mode] = (bits, lse_h)
        d = np.abs(bf16_bits_to_f64(results["fused"][0]) - bf16_bits_to_f64(results["kernel"][0]))
        assert d.max() <= 2e-2


def _with_dominant_keys(inp, where, value_bits=0x4100):
    """Overwrite the cache rows of (sequence, token) pairs in `where` with a
    constant (8.0 by default) and the queries with 1.0: those keys score
    ~2.8e2 in log2 units against ~1e1 for the others, far above the first
    visible maximum plus the kernels' headroom, so every segment holding one
    must raise its softmax reference and restart. Without that the weights
    would overflow FP32."""
    import dataclasses
    q = np.full_like(inp.q_bits, 0x3F80)            # 1.0
    kv = inp.kv_bits.copy()
    for b, t in where:
        phys = inp.block_table[b, t // 64]
        kv[phys, t % 64, 0, :] = value_bits
    return dataclasses.replace(inp, q_bits=q, kv_bits=kv)


@pytest.mark.parametrize("h_q,s_q,causal,parts", [(16, 1, False, 0), (16, 1, False, 16),
                                                  (64, 1, False, 0), (128, 2, True, 0),
                                                  (128, 2, True, 24)])
def test_reference_restart_on_dominant_key(h_q, s_q, causal, parts):
    """A key whose score exceeds the row's first maximum by far more than the
    headroom, late in the sequence (and, with splits, inside a later
    partition): the kernels raise the reference and redo the segment; the
    result must match the oracle (output ~ that key's value row)."""
    inp = make_inputs([3000, 700, 150], s_q, h_q, seed=41 + parts, causal=causal)
    inp = _with_dominant_keys(inp, [(0, 2500), (1, 600), (2, 100)])
    out, lse = _check(inp, num_partitions=parts, tag=f"restart h_q={h_q} parts={parts}")
    assert np.all(np.isfinite(lse))


@pytest.mark.parametrize("h_q,s_q,causal,parts", [(16, 1, False, 0), (16, 1, False, 16), (64, 1, False, 24)])
def test_reference_restart_fused_wave_forced(h_q, s_q, causal, parts, plan_override):
    """The redo of a segment on the fused-wave organisation when a later key
    dominates, with fewer rows than its block and with splits."""
    plan_override(kernel="fw")
    inp = make_inputs([3000, 700, 150], s_q, h_q, seed=43 + parts, causal=causal)
    inp = _with_dominant_keys(inp, [(0, 2500), (1, 600), (2, 100)])
    out, lse = _check(inp, num_partitions=parts, tag=f"restart-fw h_q={h_q} parts={parts}")
    assert np.all(np.isfinite(lse))


def test_pages_past_4_gib():
    """A 5.3 GB cache with the used pages at its top: page offsets pass 2^32
    bytes, so 32-bit address arithmetic anywhere would read the wrong rows.
    Decode, and the cache append into those pages, against the oracle on the
    same logical content."""
    import torch
    import mla_paged_kv_02_amd as mla
    from workloads import make_append_inputs
    inp = make_inputs([300, 70, 129], 2, 16, seed=91, causal=True)
    nb = inp.num_pages
    total = 72000                                       # 72000 * 73728 B = 5.3 GB
    shift = total - nb
    log(f"[case] pages past 4 GiB: cache {total} pages, used pages at {shift}..{total - 1}")
    big = torch.empty((total, 64, 1, 576), dtype=torch.bfloat16, device="cuda")
    big[shift:] = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).cuda()
    table = np.where(inp.block_table >= 0, inp.block_table + shift, -1).astype(np.int32)
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(inp.seqlens).cuda()
    out, lse = mla.decode_fwd(q, big, bt, sl, inp.scale, True)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.mla_decode_ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens,
                                             inp.scale, True)
    s = score(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref_out, ref_lse)
    log(f"  decode {s}")
    assert s.ok(), str(s)
    # append two new tokens per sequence into the top pages
    app = make_append_inputs([300, 70, 129], 2, seed=92)
    new = torch.from_numpy(app.new_bits.view(np.int16)).view(torch.bfloat16).cuda()
    mla.kv_append(new, sl, bt, big)
    torch.cuda.synchronize()
    ref_kv, _ = oracle.kv_append_ref(inp.kv_bits, app.new_bits, inp.block_table, inp.seqlens)
    got = big[shift:].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref_kv), "append into pages past 4 GiB"
    del big
    torch.cuda.empty_cache()


def test_mismatched_plan_writes_nan_lse_and_nothing_else(plan_override):
    """A plan built for other arguments, passed through the C ABI (the Python
    binding refuses it first): the decode kernel finds the header mismatch
    before it reads anything else, writes NaN into every lse entry and stores
    nothing else. Every case keeps the kernel's reads of the plan inside the
    buffer (the plan has at least as many partition records as the call)."""
    import ctypes
    import torch
    import mla_paged_kv_02_amd as mla
    from mla_paged_kv_02_amd import _lib
    from gpu_util import to_device
    from workloads import make_fp8_cache, pack_fp8_pages
    inp = make_inputs([300, 70, 129], 1, 64, seed=95)
    q, kv, bt, sl = to_device(inp)
    pages = torch.from_numpy(pack_fp8_pages(*make_fp8_cache(inp, seed=96))).cuda()
    cases = [  # (tag, plan h_q, plan partitions, call h_q, call partitions, fp8 call)
        ("partition count", 64, 128, 64, 64, False),
        ("row blocks", 64, 64, 256, 64, False),   # 1 vs 2 blocks even with 128-row blocks
        # under the default choice 32 rows take two 16-row blocks over BF16
        # and one 32-row score/value block over FP8: the plans differ (this
        # case sets the default choice whatever --decode-kernel forces)
        ("BF16 plan into the FP8 call", 32, 64, 32, 64, True),
        ("16-row plan, other partition count", 16, 64, 16, 32, False),
    ]
    for tag, ph, pp, ch, cp, fp8 in cases:
        if fp8:
            mla.set_plan_override()
        else:
            plan_override(kernel=None)
        meta = mla.get_split_metadata(sl, ph, 1, pp)
        host = meta.metadata.cpu().numpy()
        assert _lib.lib().mla_check_metadata_host(host.ctypes.data, host.nbytes, inp.batch, ch, 1, cp,
                                                  int(fp8)) == 1, tag
        qc = q if ch == 64 else torch.cat([q] * (ch // 64), dim=2).contiguous() if ch > 64 else q[:, :, :ch].contiguous()
        out = torch.full((inp.batch, 1, ch, 512), 1.5, dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros((inp.batch, 1, ch), dtype=torch.float32, device="cuda")
        ws = torch.empty(_lib.lib().mla_workspace_bytes(inp.batch, ch, 1, cp), dtype=torch.uint8, device="cuda")
        fn = _lib.lib().mla_decode_fwd_fp8 if fp8 else _lib.lib().mla_decode_fwd
        cache = pages if fp8 else kv
        log(f"[case] mismatched plan: {tag}")
        st = fn(qc.data_ptr(), cache.data_ptr(), bt.data_ptr(), bt.shape[1], sl.data_ptr(), inp.batch, 1, ch,
                cache.shape[0], ctypes.c_float(inp.scale), 0, meta.metadata.data_ptr(), cp, ws.data_ptr(),
                ws.numel(), out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == 0, tag
        assert torch.isnan(lse).all().item(), f"{tag}: lse not NaN everywhere"
        assert (out.float() == 1.5).all().item(), f"{tag}: out was written"
        # the plan itself is untouched
        assert np.array_equal(meta.metadata.cpu().numpy(), host), f"{tag}: plan changed"
