"""Absorption products on the GPU vs the oracle, through the C ABI.

Tolerance of one product (derived from the arithmetic): the bf16 x bf16
products are exact in FP32 and summed in FP32 over K terms, an error of at
most K * 2^-24 * sum_k |w_k x_k| (taken twice over, for slack in the
accumulation order), and the result is rounded once to BF16, at most 2^-8 of
its magnitude. So each element must satisfy

    |got - ref| <= 2^-8 |ref| + K * 2^-23 * sum_k |w_k x_k|.

The rotary part of the absorbed query is a copy and must match bit for bit.
The whole chain (absorb_q, decode, absorb_o) is compared with the FP64
non-absorbed chain: three BF16 roundings (2^-8 each) plus the decode gate
(relative L2 5e-3) bound its relative L2 error by about 1.7e-2; the test
asks for 2e-2.
"""

import numpy as np
import pytest

import oracle
from gpu_util import bf16_bits_to_f64, log, score
from workloads import bf16_round_bits, make_inputs

pytestmark = pytest.mark.gpu


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _bf16(rng, shape, std=1.0):
    return bf16_round_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _check_product(got_bits, ref, w, x, k, what):
    """got [T, H, M] bits; ref [T, H, M] fp64; w [H, M, K], x [T, H, K] fp64."""
    got = bf16_bits_to_f64(got_bits)
    mag = np.einsum("hmk,thk->thm", np.abs(w), np.abs(x))
    bound = 2.0 ** -8 * np.abs(ref) + k * 2.0 ** -23 * mag
    err = np.abs(got - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= bound), f"{what}: error exceeds its bound (worst ratio {worst:.2f})"
    return worst


@pytest.mark.parametrize("tokens,heads,d_nope", [(1, 1, 32), (5, 3, 96), (70, 16, 128), (130, 128, 128),
                                                 (9, 3, 128), (33, 8, 512), (64, 2, 64)])
def test_absorb_q_matches_oracle(tokens, heads, d_nope):
    import torch
    import mla_paged_kv_02_amd as mla
    log(f"[case] absorb_q T={tokens} H={heads} dn={d_nope}")
    rng = np.random.default_rng(1000 + tokens + d_nope)
    q_nope = _bf16(rng, (tokens, heads, d_nope))
    q_rope = _bf16(rng, (tokens, heads, 64))
    w_uk = _bf16(rng, (heads, 512, d_nope), 1.0 / np.sqrt(d_nope))
    out = mla.absorb_q(_dev(q_nope), _dev(q_rope), _dev(w_uk))
    torch.cuda.synchronize()
    got = _host(out)
    assert np.array_equal(got[..., 512:], q_rope), "rotary part not copied exactly"
    ref = oracle.absorb_q_ref(bf16_bits_to_f64(q_nope), bf16_bits_to_f64(q_rope), bf16_bits_to_f64(w_uk))
    worst = _check_product(got[..., :512], ref[..., :512], bf16_bits_to_f64(w_uk), bf16_bits_to_f64(q_nope),
                           d_nope, "absorb_q")
    log(f"  worst error / bound = {worst:.3f}")


@pytest.mark.parametrize("tokens,heads,d_v", [(1, 1, 32), (5, 3, 96), (70, 16, 128), (130, 128, 128),
                                              (33, 4, 512), (17, 2, 160)])
def test_absorb_o_matches_oracle(tokens, heads, d_v):
    import torch
    import mla_paged_kv_02_amd as mla
    log(f"[case] absorb_o T={tokens} H={heads} dv={d_v}")
    rng = np.random.default_rng(2000 + tokens + d_v)
    o_lat = _bf16(rng, (tokens, heads, 512))
    w_uv = _bf16(rng, (heads, 512, d_v), 1.0 / np.sqrt(512))
    w_uv_t = np.ascontiguousarray(w_uv.transpose(0, 2, 1))      # layout the kernel takes
    out = mla.absorb_o(_dev(o_lat), _dev(w_uv_t))
    torch.cuda.synchronize()
    ref = oracle.absorb_o_ref(bf16_bits_to_f64(o_lat), bf16_bits_to_f64(w_uv))
    worst = _check_product(_host(out), ref, bf16_bits_to_f64(w_uv_t), bf16_bits_to_f64(o_lat), 512, "absorb_o")
    log(f"  worst error / bound = {worst:.3f}")


@pytest.mark.parametrize("s_q,heads,causal", [(1, 16, False), (2, 128, True)])
def test_absorbed_chain_matches_nonabsorbed_form(s_q, heads, causal):
    """absorb_q -> decode -> absorb_o on the GPU against the FP64 chain on the
    same BF16 inputs; and each stage against the oracle on the GPU's own
    inputs to that stage."""
    import torch
    import mla_paged_kv_02_amd as mla
    log(f"[case] absorbed chain s_q={s_q} H={heads} causal={causal}")
    dn, dv = 128, 128
    base = make_inputs([300, 64, 7, 1200], s_q, 1, seed=80 + s_q, causal=causal)
    rng = np.random.default_rng(81 + s_q)
    B = base.batch
    q_nope = _bf16(rng, (B, s_q, heads, dn))
    q_rope = _bf16(rng, (B, s_q, heads, 64))
    w_uk = _bf16(rng, (heads, 512, dn), 1.0 / np.sqrt(dn))
    w_uv = _bf16(rng, (heads, 512, dv), 1.0 / np.sqrt(512))
    kv = _dev(base.kv_bits)
    bt = torch.from_numpy(base.block_table).cuda()
    sl = torch.from_numpy(base.seqlens).cuda()
    q_abs = mla.absorb_q(_dev(q_nope), _dev(q_rope), _dev(w_uk))
    o_lat, lse = mla.decode_fwd(q_abs, kv, bt, sl, base.scale, causal)
    out = mla.absorb_o(o_lat, _dev(np.ascontiguousarray(w_uv.transpose(0, 2, 1))))
    torch.cuda.synchronize()

    # stage by stage, each on the GPU's own input to it
    q_abs_bits = _host(q_abs)
    ref_lat, ref_lse = oracle.mla_decode_ref(q_abs_bits, base.kv_bits, base.block_table, base.seqlens,
                                             base.scale, causal)
    s = score(_host(o_lat), lse.cpu().numpy(), ref_lat, ref_lse)
    log(f"  decode on the absorbed query: {s}")
    assert s.ok(), str(s)
    o_lat_bits = _host(o_lat).reshape(B * s_q, heads, 512)
    ref_o = oracle.absorb_o_ref(bf16_bits_to_f64(o_lat_bits), bf16_bits_to_f64(w_uv))
    _check_product(_host(out).reshape(B * s_q, heads, dv), ref_o,
                   bf16_bits_to_f64(np.ascontiguousarray(w_uv.transpose(0, 2, 1))),
                   bf16_bits_to_f64(o_lat_bits), 512, "absorb_o in the chain")

    # the whole chain against FP64 throughout
    qa = oracle.absorb_q_ref(bf16_bits_to_f64(q_nope).reshape(B * s_q, heads, dn),
                             bf16_bits_to_f64(q_rope).reshape(B * s_q, heads, 64), bf16_bits_to_f64(w_uk))
    lat, _ = oracle.mla_decode_ref_f64(qa.reshape(B, s_q, heads, 576), bf16_bits_to_f64(base.kv_bits),
                                       base.block_table, base.seqlens, float(np.float32(base.scale)), causal)
    full = oracle.absorb_o_ref(lat.reshape(B * s_q, heads, 512), bf16_bits_to_f64(w_uv))
    got = bf16_bits_to_f64(_host(out)).reshape(B * s_q, heads, dv)
    rel = float(np.linalg.norm(got - full) / np.linalg.norm(full))
    log(f"  whole chain relative L2 {rel:.2e}")
    assert rel <= 2e-2
