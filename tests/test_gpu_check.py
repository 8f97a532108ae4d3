"""mla_check_decode_inputs on the GPU: the count of decode-precondition
violations (lengths outside [0, 64 * max_blocks], table entries the decode
reads outside [0, num_pages)) is exact, entries past a sequence's last page
are ignored, and valid workloads count zero. The expected counts follow the
definition directly on the host; nothing here comes from the HIP path."""

import numpy as np
import pytest
import torch

from gpu_util import log

pytestmark = pytest.mark.gpu


def _count(bt, seqlens, num_pages):
    import mla_paged_kv_02_amd as mla
    dev = torch.device("cuda:0")
    v = mla.check_decode_inputs(torch.from_numpy(bt).to(dev), torch.from_numpy(seqlens).to(dev), num_pages)
    torch.cuda.synchronize()
    return int(v.item())


def _expected(bt, seqlens, num_pages):
    bad = 0
    for b, n in enumerate(seqlens.tolist()):
        if n < 0 or n > 64 * bt.shape[1]:
            bad += 1
            continue
        row = bt[b, :(n + 63) // 64]
        bad += int(((row < 0) | (row >= num_pages)).sum())
    return bad


def _valid(batch, max_blocks, seed):
    rng = np.random.default_rng(seed)
    seqlens = rng.integers(0, 64 * max_blocks + 1, batch).astype(np.int32)
    need = (seqlens + 63) // 64
    num_pages = int(need.sum()) + 3
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((batch, max_blocks), -1, dtype=np.int32)
    k = 0
    for b in range(batch):
        bt[b, :need[b]] = perm[k:k + need[b]]
        # entries past the last page: garbage the decode never reads
        bt[b, need[b]:] = rng.choice([-1, np.iinfo(np.int32).max, num_pages, -7], max_blocks - need[b])
        k += need[b]
    return bt, seqlens, num_pages


@pytest.mark.parametrize("batch,max_blocks", [(1, 1), (7, 5), (64, 80), (3000, 9)])
def test_valid_inputs_count_zero(batch, max_blocks):
    log(f"[case] check_decode_inputs valid B={batch} max_blocks={max_blocks}")
    bt, seqlens, num_pages = _valid(batch, max_blocks, seed=batch + max_blocks)
    assert _expected(bt, seqlens, num_pages) == 0
    assert _count(bt, seqlens, num_pages) == 0


def test_planted_violations_are_counted_exactly():
    log("[case] check_decode_inputs planted violations")
    bt, seqlens, num_pages = _valid(50, 12, seed=7)
    rng = np.random.default_rng(8)
    live = [(b, n) for b in range(50) for n in range((int(seqlens[b]) + 63) // 64)]
    picks = rng.choice(len(live), 9, replace=False)
    for i, p in enumerate(picks):
        b, n = live[p]
        bt[b, n] = [-1, num_pages, num_pages + 1000, np.iinfo(np.int32).min][i % 4]
    seqlens[3] = -5                      # negative length: one violation, entries unchecked
    seqlens[4] = 64 * 12 + 1             # one token past the table
    seqlens[5] = 64 * 12                 # exactly full: valid
    need5 = 12
    bt[5, :need5] = rng.integers(0, num_pages, need5)
    exp = _expected(bt, seqlens, num_pages)
    assert exp >= 2
    assert _count(bt, seqlens, num_pages) == exp


def test_named_workload_counts_zero():
    from workloads import make_workload_inputs
    inp = make_workload_inputs("memory_bound")
    log("[case] check_decode_inputs memory_bound workload")
    nb = int(inp.kv_bits.shape[0])
    assert _count(np.ascontiguousarray(inp.block_table), np.ascontiguousarray(inp.seqlens), nb) == 0
    bt = np.ascontiguousarray(inp.block_table).copy()
    bt[10, 0] = nb   # one page past the cache
    assert _count(bt, np.ascontiguousarray(inp.seqlens), nb) == 1
