"""Paged grouped-query MHA decode (the contrast case) on the GPU vs the
oracle, through the C ABI, with the decode gates."""

import dataclasses

import numpy as np
import pytest

import oracle
from gpu_util import log, score
from workloads import make_mha_inputs, make_mha_workload

pytestmark = pytest.mark.gpu


def _run(inp):
    import torch
    import mla_paged_kv_02_amd as mla
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = mla.mha_decode_fwd(dev(inp.q_bits), dev(inp.k_bits), dev(inp.v_bits),
                                  torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seqlens).cuda(),
                                  inp.scale, inp.causal)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def _check(inp, tag, seqs=None):
    log(f"[case] mha {tag} B={inp.batch} q={inp.q_bits.shape} kv={inp.k_bits.shape} causal={inp.causal}")
    out, lse = _run(inp)
    sub = inp
    if seqs is not None:
        sub = dataclasses.replace(inp, q_bits=inp.q_bits[seqs], block_table=inp.block_table[seqs],
                                  seqlens=inp.seqlens[seqs])
    ref_out, ref_lse = oracle.mha_decode_ref(sub.q_bits, sub.k_bits, sub.v_bits, sub.block_table, sub.seqlens,
                                             sub.scale, sub.causal)
    if seqs is not None:
        out, lse = out[seqs], lse[seqs]
    s = score(out, lse, ref_out, ref_lse)
    log(f"  {s}")
    assert s.ok(), str(s)
    return out, lse


MHA_CASES = [
    # (seqlens, s_q, h_q, h_kv, causal)
    ([37, 100], 1, 16, 8, False),
    ([1, 63, 64, 65, 127, 129, 300], 1, 16, 8, False),
    ([0, 5, 0, 200], 1, 8, 8, False),
    ([700, 1], 1, 16, 1, False),
    ([130, 257, 64], 2, 8, 2, True),
    ([3, 70, 129], 4, 4, 1, True),
]


@pytest.mark.parametrize("case", range(len(MHA_CASES)))
def test_mha_small_shapes(case):
    seqlens, s_q, h_q, h_kv, causal = MHA_CASES[case]
    _check(make_mha_inputs(seqlens, s_q, h_q, h_kv, 128, seed=500 + case, causal=causal), f"small[{case}]")


def test_mha_poisoned_tails_are_ignored():
    inp = make_mha_inputs([70, 5, 129, 64], 1, 16, 8, 128, seed=510)
    out0, lse0 = _check(inp, "clean")
    k, v = inp.k_bits.copy(), inp.v_bits.copy()
    for b, n in enumerate(inp.seqlens):
        n = int(n)
        if n % 64:
            phys = int(inp.block_table[b, n // 64])
            k[phys, n % 64:] = 0x7FC0
            v[phys, n % 64:] = 0x7FC0
    out1, lse1 = _run(dataclasses.replace(inp, k_bits=k, v_bits=v))
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_mha_workload_full_size():
    inp = make_mha_workload("mha_memory_bound")
    _check(inp, "mha_memory_bound")


def test_mha_rejects_groups_over_16_rows():
    import torch
    import mla_paged_kv_02_amd as mla
    inp = make_mha_inputs([10], 2, 16, 1, 128, seed=520)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    with pytest.raises(mla.MlaError, match="UNSUPPORTED"):
        mla.mha_decode_fwd(dev(inp.q_bits), dev(inp.k_bits), dev(inp.v_bits), torch.from_numpy(inp.block_table).cuda(),
                           torch.from_numpy(inp.seqlens).cuda(), inp.scale, False)


def test_mha_pages_past_4_gib():
    """Key and value pages at the top of 4.3 GB caches (offsets past 2^32)."""
    import torch
    import mla_paged_kv_02_amd as mla
    inp = make_mha_inputs([300, 70, 129], 1, 16, 8, 128, seed=530)
    nb = inp.k_bits.shape[0]
    total = 33000                                   # 33000 * 131072 B = 4.3 GB each
    shift = total - nb
    log(f"[case] mha pages past 4 GiB: {total} pages, used at {shift}..")
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    k = torch.empty((total, 64, 8, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    k[shift:] = dev(inp.k_bits)
    v[shift:] = dev(inp.v_bits)
    table = np.where(inp.block_table >= 0, inp.block_table + shift, -1).astype(np.int32)
    out, lse = mla.mha_decode_fwd(dev(inp.q_bits), k, v, torch.from_numpy(table).cuda(),
                                  torch.from_numpy(inp.seqlens).cuda(), inp.scale, False)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.mha_decode_ref(inp.q_bits, inp.k_bits, inp.v_bits, inp.block_table, inp.seqlens,
                                             inp.scale, False)
    s = score(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref_out, ref_lse)
    log(f"  {s}")
    assert s.ok(), str(s)
    del k, v
    torch.cuda.empty_cache()
