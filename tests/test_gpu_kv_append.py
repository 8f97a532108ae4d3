"""Paged cache append on the GPU vs the oracle, through the C ABI.

The whole cache is compared bit for bit after the call (so rows that must not
change are checked too), and the count of tokens without a page must match.
Then decode runs on the appended cache with the new tokens as its causal
queries and is scored against the oracle decode over the oracle's cache.
"""

import numpy as np
import pytest

import oracle
import oracle_pins as P
from gpu_util import log, score
from workloads import APPEND_WORKLOADS, make_append_inputs, make_append_workload, make_inputs

pytestmark = pytest.mark.gpu


def _bits_to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_append(inp, count=True):
    import torch
    import mla_paged_kv_02_amd as mla
    kv = _bits_to_dev(inp.kv_bits)
    new = _bits_to_dev(inp.new_bits)
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).cuda()
    sl = torch.from_numpy(inp.seqlens).cuda()
    skipped = torch.zeros((), dtype=torch.int32, device="cuda") if count else None
    mla.kv_append(new, sl, bt, kv, skipped)
    torch.cuda.synchronize()
    kv_bits = kv.view(torch.int16).cpu().numpy().view(np.uint16)
    return kv_bits, (int(skipped.item()) if count else None)


def _check_append(inp, tag, count=True):
    log(f"[case] append {tag} B={inp.batch} s_new={inp.s_new} pages={inp.kv_bits.shape[0]} "
        f"width={inp.block_table.shape[1]}")
    got, skipped = _run_append(inp, count)
    ref, ref_skipped = oracle.kv_append_ref(inp.kv_bits, inp.new_bits, inp.block_table, inp.seqlens)
    diff = np.argwhere(np.any(got != ref, axis=-1))
    assert diff.size == 0, f"{len(diff)} cache rows differ, first (page, slot): {diff[:4].tolist()}"
    if count:
        assert skipped == ref_skipped, f"skipped {skipped}, oracle {ref_skipped}"
    return ref_skipped


@pytest.mark.parametrize("s_new", [1, 3, 64, 70, 130])
def test_append_ragged_lengths(s_new):
    inp = make_append_inputs([0, 1, 5, 63, 64, 65, 128, 130, 200, 333], s_new, seed=50 + s_new,
                             extra_blocks=1)
    assert _check_append(inp, f"ragged s_new={s_new}") == 0


def test_append_table_holes_are_counted_not_written():
    # the same three kinds of hole as the oracle's physical-view pin: a -1
    # entry, an entry past the cache, and a table row too narrow for its sequence
    cases = P._append_cases(seed=60)
    total = 0
    for k, inp in enumerate(cases):
        total += _check_append(inp, f"holes[{k}]")
    assert total > 0


def test_append_without_counter():
    inp = P._append_cases(seed=61)[1]
    _check_append(inp, "holes, no counter", count=False)


def test_append_sequences_shorter_than_new_tokens():
    inp = make_append_inputs([0, 2, 7], 40, seed=62)
    assert _check_append(inp, "all short") == 0


@pytest.mark.parametrize("name", sorted(APPEND_WORKLOADS))
def test_append_workload_full_size(name):
    inp = make_append_workload(name)
    assert _check_append(inp, name) == 0


@pytest.mark.parametrize("h_q,s_q", [(16, 4), (128, 2), (16, 64)])
def test_append_then_causal_decode(h_q, s_q):
    """Append s_q new rows, then decode those s_q tokens causally over the
    appended cache; the cache must equal the oracle's and decode must pass the
    usual gates against the oracle decode on that cache."""
    import torch
    import mla_paged_kv_02_amd as mla
    seqlens = [300, 64, 2, 129, 1000]
    dec = make_inputs(seqlens, s_q, h_q, seed=70 + s_q, causal=True)
    app = make_append_inputs(seqlens, s_q, seed=71 + s_q)
    # decode's pages and table, the append's new rows; the cache before the
    # append holds poison where the new rows go, so a missed row shows
    kv_before, _ = oracle.kv_append_ref(dec.kv_bits, np.full_like(app.new_bits, 0x7FC0),
                                        dec.block_table, dec.seqlens)
    ref_kv, _ = oracle.kv_append_ref(kv_before, app.new_bits, dec.block_table, dec.seqlens)
    log(f"[case] append+decode h_q={h_q} s_q={s_q}")
    kv = _bits_to_dev(kv_before)
    new = _bits_to_dev(app.new_bits)
    q = _bits_to_dev(dec.q_bits)
    bt = torch.from_numpy(dec.block_table).cuda()
    sl = torch.from_numpy(dec.seqlens).cuda()
    mla.kv_append(new, sl, bt, kv)
    meta = mla.get_split_metadata(sl, h_q, s_q)
    out, lse = mla.decode_fwd(q, kv, bt, sl, dec.scale, True, meta=meta)
    torch.cuda.synchronize()
    got_kv = kv.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_kv, ref_kv)
    ref_out, ref_lse = oracle.mla_decode_ref(dec.q_bits, ref_kv, dec.block_table, dec.seqlens,
                                             dec.scale, True)
    s = score(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref_out, ref_lse)
    log(f"  {s}")
    assert s.ok(), str(s)
