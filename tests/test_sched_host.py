"""Split-KV plan invariants, checked on the host build of the scheduler.

The plan is not unique (any partition of the page list is correct), so it is
pinned by invariants: every (sequence, page) pair is covered exactly once,
ranges are contiguous and ordered, split counts and partial slots agree with
the ranges, and no partition costs more than its share plus one segment.
"""

import numpy as np
import pytest

from mla_paged_kv_02_amd import split_metadata_host

HEADER = 16
PART_INTS = 8   # b_begin, n_begin, b_end, n_end, length of b_begin, 3 zeros


def decode_plan(meta, batch):
    P = int(meta[2])
    rec = meta[HEADER:HEADER + PART_INTS * P].reshape(P, PART_INTS)
    parts = rec[:, :4]
    seq = meta[HEADER + PART_INTS * P:HEADER + PART_INTS * P + 4 * batch].reshape(batch, 4)
    return dict(magic=int(meta[0]), batch=int(meta[1]), P=P, cseg=int(meta[3]), W=int(meta[4]),
                slots=int(meta[5]), total=int(meta[6]), active=int(meta[7]), parts=parts, seq=seq,
                first_len=rec[:, 4], pad=rec[:, 5:])


def segments(plan, seqlens):
    """(partition, b, lo, hi) for every non-empty page range, walking each
    partition the way the decode kernel does."""
    pages = (np.asarray(seqlens) + 63) // 64
    out = []
    for p, (b0, n0, b1, n1) in enumerate(plan["parts"]):
        b = b0
        while b < b1 or (b == b1 and n1 > 0):
            if b >= len(seqlens):
                break
            lo = n0 if b == b0 else 0
            hi = n1 if b == b1 else pages[b]
            if hi > lo:
                out.append((p, b, lo, hi))
            b += 1
    return out


def check_plan(seqlens, h_q=16, s_q=1, nparts=64):
    seqlens = np.asarray(seqlens, dtype=np.int32)
    meta = split_metadata_host(seqlens, h_q, s_q, nparts)
    plan = decode_plan(meta, len(seqlens))
    assert plan["magic"] == 0x314C4D41 and plan["batch"] == len(seqlens)
    assert plan["P"] % 8 == 0 and plan["P"] >= nparts
    pages = (seqlens.astype(np.int64) + 63) // 64
    segs = segments(plan, seqlens)

    # every page exactly once
    cover = [np.zeros(n, dtype=np.int64) for n in pages]
    for p, b, lo, hi in segs:
        cover[b][lo:hi] += 1
    for b in range(len(seqlens)):
        assert np.all(cover[b] == 1), f"sequence {b} covered {cover[b]}"

    # partitions are ordered along the page list and contiguous
    flat = [(b, n) for p, b, lo, hi in segs for n in range(lo, hi)]
    assert flat == [(b, n) for b in range(len(seqlens)) for n in range(pages[b])]

    # per-sequence split bookkeeping
    slot = 0
    for b in range(len(seqlens)):
        parts_b = sorted({p for p, bb, lo, hi in segs if bb == b})
        base, first, count, _start = plan["seq"][b]
        if pages[b] == 0:
            assert first == -1 and count == 0 and base == -1
            continue
        assert parts_b == list(range(first, first + count))
        if count > 1:
            assert base == slot
            slot += count
        else:
            assert base == -1
    assert plan["slots"] == slot <= 2 * plan["P"]
    assert plan["active"] == min(plan["P"], plan["total"])
    for p in range(plan["active"], plan["P"]):
        assert not any(s[0] == p for s in segs), "inactive partition got work"

    # each record carries its first sequence's length (0 past the batch)
    for p, (b0, _n0, _b1, _n1) in enumerate(plan["parts"]):
        assert plan["first_len"][p] == (seqlens[b0] if b0 < len(seqlens) else 0)
    assert not np.any(plan["pad"])

    # balance: no partition costs more than its share plus one extra segment
    cost = np.zeros(plan["P"], dtype=np.int64)
    for p, b, lo, hi in segs:
        cost[p] += (hi - lo) + plan["cseg"]
    assert cost.max() <= plan["W"] + plan["cseg"], (cost.max(), plan["W"], plan["cseg"])
    return plan, segs


@pytest.mark.parametrize("seed", range(20))
def test_random_lengths(seed):
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(1, 300))
    seqlens = rng.integers(0, 20000, size=batch)
    seqlens[rng.random(batch) < 0.2] = 0            # empty sequences
    seqlens[rng.random(batch) < 0.1] = 64           # exact pages
    nparts = int(rng.integers(1, 600))
    h_q, s_q = [(16, 1), (64, 1), (128, 1), (128, 2), (32, 1)][seed % 5]
    check_plan(seqlens, h_q, s_q, nparts)


@pytest.mark.parametrize("seqlens", [
    [0], [1], [0, 0, 0], [64], [65], [1, 0, 1], [65536] * 4, [1024, 16384, 32768, 65536],
    [37, 100], list(range(0, 700, 7)),
])
def test_edge_lengths(seqlens):
    for nparts in (1, 8, 64, 256, 1000):
        check_plan(seqlens, nparts=nparts)


def test_long_context_spreads_over_partitions():
    plan, segs = check_plan([1024, 16384, 32768, 65536], h_q=64, nparts=256)
    used = {p for p, *_ in segs}
    assert len(used) >= 250            # nearly every partition has work


def test_deterministic_and_independent_of_values():
    a = split_metadata_host([100, 200, 5000], 16, 1, 64)
    b = split_metadata_host([100, 200, 5000], 16, 1, 64)
    assert np.array_equal(a, b)
