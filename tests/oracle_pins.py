"""Checks that tie the FP64 oracle to the pages and to mathematics.

Each ``pin_*`` function takes a decode function with the signature of
``oracle.mla_decode_ref`` (BF16 bit inputs) or ``oracle.mla_decode_ref_f64``
and raises AssertionError when it disagrees with a fact fixed outside the
oracle. They are collected as tests in ``test_oracle_pins.py`` and reused by
``test_oracle_mutations.py``, which plants mistakes in the oracle and checks
that some pin catches each one.
"""

from __future__ import annotations

import math

import numpy as np

import oracle
from workloads import make_inputs, permute_pages, bf16_bits_to_f32

PAGE = 64


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _paged(rows: np.ndarray, seed: int, extra_pages: int = 2):
    """Place logical rows [N, 576] (float64) into shuffled pages; returns
    kv [NB, 64, 1, 576], block_table [1, nb]. Unused slots hold NaN so any
    read past N shows up."""
    n = rows.shape[0]
    nb = (n + PAGE - 1) // PAGE
    total = nb + extra_pages
    rng = np.random.default_rng(seed)
    perm = rng.permutation(total)[:nb]
    kv = np.full((total, PAGE, 1, rows.shape[1]), np.nan)
    for t in range(n):
        kv[perm[t // PAGE], t % PAGE, 0] = rows[t]
    return kv, perm[None, :].astype(np.int32)


# (a) Non-absorbed identity: the MLA page's up-projected form equals the
# absorbed form used by decode (q_abs = [W_UK q_nope ; q_rope], o = o_lat W_UV).
def pin_nonabsorbed_identity(ref_f64, seed=11, n=150, heads=4, dn=128, dv=96):
    rng = np.random.default_rng(seed)
    c_kv = rng.standard_normal((n, 512))
    k_rope = rng.standard_normal((n, 64))
    w_uk = rng.standard_normal((heads, 512, dn)) / math.sqrt(512)
    w_uv = rng.standard_normal((heads, 512, dv)) / math.sqrt(512)
    q_nope = rng.standard_normal((heads, dn))
    q_rope = rng.standard_normal((heads, 64))
    scale = 1.0 / math.sqrt(576)
    o_ref, lse_ref = oracle.mla_nonabsorbed_ref(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, scale)

    q_abs = np.concatenate([np.einsum("hcd,hd->hc", w_uk, q_nope), q_rope], axis=1)
    kv, table = _paged(np.concatenate([c_kv, k_rope], axis=1), seed)
    out, lse = ref_f64(q_abs[None, None], kv, table, np.array([n]), scale, False)
    o_abs = np.einsum("hc,hcv->hv", out[0, 0], w_uv)
    rel = np.abs(o_abs - o_ref).max() / np.abs(o_ref).max()
    assert rel < 1e-12, f"absorbed vs non-absorbed output rel err {rel}"
    assert np.abs(lse[0, 0] - lse_ref).max() < 1e-12, "absorbed vs non-absorbed lse"


# (b) Page placement does not matter: moving physical pages and rewriting the
# block table leaves the logical sequences, hence the result, unchanged.
def pin_page_permutation(ref, seed=12):
    inp = make_inputs([37, 100, 64, 129], s_q=2, h_q=16, seed=seed, causal=True, extra_blocks=1)
    out0, lse0 = ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens, inp.scale, True)
    moved = permute_pages(inp, seed + 1)
    out1, lse1 = ref(moved.q_bits, moved.kv_bits, moved.block_table, moved.seqlens, moved.scale, True)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1), "page permutation changed result"


# (c) One cached token: softmax weight 1, so out = V_0 and lse = scale <q, K_0>.
def pin_single_token(ref, seed=13):
    inp = make_inputs([1, 1, 1], s_q=1, h_q=16, seed=seed)
    out, lse = ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens, inp.scale, False)
    for b in range(3):
        k0 = _f64(inp.kv_bits[inp.block_table[b, 0], 0, 0])
        q = _f64(inp.q_bits[b, 0])
        assert np.array_equal(out[b, 0], np.broadcast_to(k0[:512], (16, 512))), "out != V_0"
        s = float(np.float32(inp.scale)) * np.array([math.fsum(q[h] * k0) for h in range(16)])
        assert np.abs(lse[b, 0] - s).max() < 1e-12, "lse != scale <q,K_0>"


# (d) Equal scores: with q's latent part zero and one shared rotary key, all
# scores equal c, so out = mean of V and lse = c + ln N. With q = 0, lse = ln N.
def pin_equal_scores(ref_f64, seed=14, n=150):
    rng = np.random.default_rng(seed)
    latent = rng.standard_normal((n, 512))
    rope = rng.standard_normal(64)
    rows = np.concatenate([latent, np.broadcast_to(rope, (n, 64))], axis=1)
    kv, table = _paged(rows, seed)
    q = np.zeros((1, 1, 3, 576))
    q[0, 0, 1, 512:] = rng.standard_normal(64)
    q[0, 0, 2, 512:] = rng.standard_normal(64)
    scale = 1.0 / 24.0
    out, lse = ref_f64(q, kv, table, np.array([n]), scale, False)
    mean_v = latent.mean(axis=0)
    for h in range(3):
        c = scale * math.fsum(q[0, 0, h, 512:] * rope)
        assert abs(lse[0, 0, h] - (c + math.log(n))) < 1e-12, "lse != c + ln N"
        assert np.abs(out[0, 0, h] - mean_v).max() < 1e-12, "out != mean V"


# (e) Causal reductions: with s_q = 2 under the causal mask, token 1 equals a
# single-token decode over all N keys and token 0 one over the first N-1;
# with s_q = 1 the causal mask changes nothing.
def pin_causal_reductions(ref, seed=15):
    inp = make_inputs([1, 2, 64, 65, 130], s_q=2, h_q=16, seed=seed, causal=True)
    out, lse = ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens, inp.scale, True)
    for i in (0, 1):
        lens = np.maximum(inp.seqlens - (1 - i), 0).astype(np.int32)
        o1, l1 = ref(inp.q_bits[:, i:i + 1], inp.kv_bits, inp.block_table, lens, inp.scale, False)
        assert np.array_equal(out[:, i], o1[:, 0]), f"causal token {i} output"
        assert np.array_equal(lse[:, i], l1[:, 0]), f"causal token {i} lse"
    # the sequence of length 1 has no visible key for token 0
    assert np.all(np.isneginf(lse[0, 0])) and not np.any(out[0, 0]), "empty causal row"
    single = make_inputs([5, 70], s_q=1, h_q=16, seed=seed + 1)
    a = ref(single.q_bits, single.kv_bits, single.block_table, single.seqlens, single.scale, True)
    b = ref(single.q_bits, single.kv_bits, single.block_table, single.seqlens, single.scale, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "causal s_q=1 not a no-op"


# (f) Combine identity: attending over random disjoint key chunks and merging
# with the log-sum-exp rule reproduces attention over all keys.
def pin_combine_identity(attend, combine, seed=16, n=300, rows=8):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, 576))
    q = rng.standard_normal((rows, 576))
    scale = 1.0 / 24.0
    o_full, l_full = attend(q, k, [n] * rows, scale)
    cuts = np.sort(rng.choice(np.arange(1, n), size=5, replace=False))
    bounds = [0, *cuts.tolist(), n]
    parts_o, parts_l = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        o, l = attend(q, k[lo:hi], [hi - lo] * rows, scale)
        parts_o.append(o)
        parts_l.append(l)
    # an empty chunk carries no weight
    parts_o.append(np.zeros((rows, 512)))
    parts_l.append(np.full(rows, -np.inf))
    o, l = combine(np.stack(parts_o), np.stack(parts_l))
    assert np.abs(o - o_full).max() < 1e-13 and np.abs(l - l_full).max() < 1e-13, "combine"
    o_e, l_e = combine(np.zeros((2, 3, 512)), np.full((2, 3), -np.inf))
    assert not np.any(o_e) and np.all(np.isneginf(l_e)), "combine of empty parts"


# (i) Brute force: pure-Python loops with exactly rounded sums on tiny inputs.
def pin_bruteforce(ref_f64, seed=17):
    for causal in (False, True):
        inp = make_inputs([3, 70, 1], s_q=2, h_q=2, seed=seed + causal, causal=causal)
        q, kv = _f64(inp.q_bits), _f64(inp.kv_bits)
        o_bf, l_bf = oracle.mla_decode_bruteforce(q, kv, inp.block_table, inp.seqlens,
                                                  float(np.float32(inp.scale)), causal)
        o, l = ref_f64(q, kv, inp.block_table, inp.seqlens, float(np.float32(inp.scale)), causal)
        assert np.abs(o - o_bf).max() < 1e-12, "output vs brute force"
        fin = np.isfinite(l_bf)
        assert np.array_equal(fin, np.isfinite(l)), "empty rows vs brute force"
        assert np.abs(l[fin] - l_bf[fin]).max() < 1e-12, "lse vs brute force"


# (j) Bounds: max_t s_t <= lse <= max_t s_t + ln L, and every output is a
# convex combination of value rows (inside their per-column range).
def pin_bounds(ref, seed=18):
    inp = make_inputs([40, 200], s_q=1, h_q=16, seed=seed)
    out, lse = ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens, inp.scale, False)
    for b, n in enumerate(inp.seqlens):
        rows = np.stack([_f64(inp.kv_bits[inp.block_table[b, t // PAGE], t % PAGE, 0]) for t in range(n)])
        q = _f64(inp.q_bits[b, 0])
        s = float(np.float32(inp.scale)) * (q @ rows.T)
        smax = s.max(axis=1)
        assert np.all(lse[b, 0] >= smax - 1e-12) and np.all(lse[b, 0] <= smax + math.log(n) + 1e-12), "lse bounds"
        lo, hi = rows[:, :512].min(axis=0), rows[:, :512].max(axis=0)
        assert np.all(out[b, 0] >= lo - 1e-12) and np.all(out[b, 0] <= hi + 1e-12), "convexity"


# (k) Two keys, worked by hand: with scores s0, s1 the weights are the
# logistic function of their difference.
def pin_two_keys(ref_f64):
    rows = np.zeros((2, 576))
    rows[0, 0], rows[1, 0] = 1.0, -1.0        # V_0 = e_0, V_1 = -e_0
    rows[0, 1], rows[1, 1] = 2.0, 5.0         # second latent coordinate
    rows[:, 512] = [3.0, 1.0]                 # rotary coordinate
    q = np.zeros((1, 1, 1, 576))
    q[0, 0, 0, 512] = 1.0                     # s_t = scale * rope_t
    kv, table = _paged(rows, 3)
    scale = 0.5
    out, lse = ref_f64(q, kv, table, np.array([2]), scale, False)
    s0, s1 = 1.5, 0.5
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert abs(lse[0, 0, 0] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-15
    assert abs(out[0, 0, 0, 0] - (2 * w0 - 1)) < 1e-15
    assert abs(out[0, 0, 0, 1] - (2 * w0 + 5 * (1 - w0))) < 1e-14
    assert not np.any(out[0, 0, 0, 2:])


# (k) Cache append, checked from the physical side: walk every block-table
# entry and every slot of the page it names, work out which new token (if
# any) the placement rule sends there, and require that row and nothing else
# to change. Tokens with a position but no page are counted.
def _append_cases(seed):
    from workloads import make_append_inputs
    cases = []
    # ragged lengths around page edges; s_new larger than some sequences
    a = make_append_inputs([0, 1, 5, 63, 64, 65, 130, 200], 70, seed, extra_blocks=1)
    cases.append(a)
    # holes in the table: a missing page (-1), an index past the cache, and a
    # row too narrow for its sequence
    b = make_append_inputs([150, 90, 300], 80, seed + 1)
    t = b.block_table.copy()
    t[0, 1] = -1
    t[1, 0] = b.kv_bits.shape[0] + 3
    b = type(b)(b.seqlens, t, b.kv_bits, b.new_bits)
    cases.append(b)
    c = make_append_inputs([100, 260], 40, seed + 2)
    c = type(c)(c.seqlens, np.ascontiguousarray(c.block_table[:, :3]), c.kv_bits, c.new_bits)
    cases.append(c)
    return cases


def pin_append_physical_view(append, seed=30):
    for inp in _append_cases(seed):
        kv_after, skipped = append(inp.kv_bits, inp.new_bits, inp.block_table, inp.seqlens)
        expected = inp.kv_bits.copy()
        num_pages = inp.kv_bits.shape[0]
        s_new = inp.new_bits.shape[1]
        written = 0
        for b in range(inp.block_table.shape[0]):
            first_new = int(inp.seqlens[b]) - s_new   # position of new token 0
            for logical in range(inp.block_table.shape[1]):
                page = int(inp.block_table[b, logical])
                if not 0 <= page < num_pages:
                    continue
                for slot in range(PAGE):
                    i = logical * PAGE + slot - first_new
                    if 0 <= i < s_new:
                        expected[page, slot, 0] = inp.new_bits[b, i]
                        written += 1
        placed = sum(min(int(n), s_new) for n in inp.seqlens)
        assert np.array_equal(kv_after, expected), "append changed the wrong cache rows"
        assert skipped == placed - written, f"skipped {skipped}, expected {placed - written}"


# (l) Round trip: knock out the last s_new rows of every sequence in a full
# cache and append them again; the cache must come back bit for bit, and
# decode over it must match decode over the original.
def pin_append_round_trip(append, seed=31, s_new=9):
    inp = make_inputs([300, 64, 7, 129, 9], 1, 4, seed)
    kv = inp.kv_bits
    new = np.zeros((inp.batch, s_new, kv.shape[-1]), dtype=np.uint16)
    damaged = kv.copy()
    for b, n in enumerate(inp.seqlens):
        n = int(n)
        rows = oracle.gather_sequence_rows(kv, inp.block_table[b], n)
        for i in range(s_new):
            pos = n - s_new + i
            if pos < 0:
                new[b, i] = 0x3F80    # no place: must not be written anywhere
                continue
            new[b, i] = rows[pos]
            damaged[inp.block_table[b, pos // PAGE], pos % PAGE, 0] = 0x7FC0
    restored, skipped = append(damaged, new, inp.block_table, inp.seqlens)
    assert skipped == 0
    assert np.array_equal(restored, kv), "round trip did not restore the cache"
    out0, lse0 = oracle.mla_decode_ref(inp.q_bits, kv, inp.block_table, inp.seqlens, inp.scale, False)
    out1, lse1 = oracle.mla_decode_ref(inp.q_bits, restored, inp.block_table, inp.seqlens, inp.scale, False)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


# (m) Absorption, end to end: absorbing W_UK into the query, decoding over the
# latent cache and applying W_UV afterwards equals the non-absorbed MLA form
# (keys and values up-projected from the cache per head, then attention), for
# several tokens with their own queries and head widths unlike 512.
def pin_absorb_end_to_end(absorb_q, absorb_o, ref_f64, seed=32, n=130, heads=3, dn=96, dv=80):
    rng = np.random.default_rng(seed)
    c_kv = rng.standard_normal((n, 512))
    k_rope = rng.standard_normal((n, 64))
    w_uk = rng.standard_normal((heads, 512, dn)) / math.sqrt(512)
    w_uv = rng.standard_normal((heads, 512, dv)) / math.sqrt(512)
    tokens = 2
    q_nope = rng.standard_normal((tokens, heads, dn))
    q_rope = rng.standard_normal((tokens, heads, 64))
    scale = 1.0 / math.sqrt(576)
    q_abs = absorb_q(q_nope, q_rope, w_uk)                       # [T, H, 576]
    kv, table = _paged(np.concatenate([c_kv, k_rope], axis=1), seed)
    out_lat, _ = ref_f64(q_abs[None], kv, table, np.array([n]), scale, False)   # s_q = T
    o = absorb_o(out_lat[0], w_uv)                               # [T, H, dv]
    for t in range(tokens):
        o_ref, _ = oracle.mla_nonabsorbed_ref(c_kv, k_rope, q_nope[t], q_rope[t], w_uk, w_uv, scale)
        rel = np.abs(o[t] - o_ref).max() / np.abs(o_ref).max()
        assert rel < 1e-12, f"token {t}: absorbed chain vs non-absorbed rel err {rel}"


# (n) Selection weights: with W_UK_h placing q_nope coordinate d at latent
# column sigma_h(d) (a 0/1 matrix) the absorbed query is q_nope scattered to
# those columns, zero elsewhere, followed by q_rope; with W_UV_h picking
# latent column tau_h(v) for output v the output gathers those columns.
def pin_absorb_selection(absorb_q, absorb_o, seed=33, heads=3, dn=40, dv=24):
    rng = np.random.default_rng(seed)
    tokens = 5
    q_nope = rng.standard_normal((tokens, heads, dn))
    q_rope = rng.standard_normal((tokens, heads, 64))
    o_lat = rng.standard_normal((tokens, heads, 512))
    w_uk = np.zeros((heads, 512, dn))
    w_uv = np.zeros((heads, 512, dv))
    sig = [rng.choice(512, size=dn, replace=False) for _ in range(heads)]
    tau = [rng.choice(512, size=dv, replace=False) for _ in range(heads)]
    for h in range(heads):
        w_uk[h, sig[h], np.arange(dn)] = 1.0
        w_uv[h, tau[h], np.arange(dv)] = 1.0
    q_abs = absorb_q(q_nope, q_rope, w_uk)
    o = absorb_o(o_lat, w_uv)
    for h in range(heads):
        expect = np.zeros((tokens, 512))
        expect[:, sig[h]] = q_nope[:, h, :]
        assert np.array_equal(q_abs[:, h, :512], expect), f"head {h}: absorbed query"
        assert np.array_equal(q_abs[:, h, 512:], q_rope[:, h, :]), f"head {h}: rotary part"
        assert np.array_equal(o[:, h, :], o_lat[:, h, tau[h]]), f"head {h}: output"


# (o) E4M3 values fixed by the OCP 8-bit floating point specification: zero
# and negative zero, the smallest subnormal 2^-9, the largest subnormal
# 7 * 2^-9, the smallest normal 2^-6, one, one and a half, the largest
# normal 448, NaN only at S.1111.111, and 254 finite values increasing with
# the code within each sign.
def pin_e4m3_table(decode):
    v = decode(np.arange(256, dtype=np.uint8))
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in fixed.items():
        assert v[code] == val, f"E4M3 0x{code:02x} = {v[code]}, expected {val}"
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0, "0x80 must be -0"
    nan = np.isnan(v)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}, "NaN codes"
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes not increasing"
    assert np.array_equal(v[0x80:0xFF], -pos), "negative codes are not the mirror"


# (p) Quantiser: the largest magnitude of a row lands on +-448 exactly; a row
# made of E4M3 values times a power of two comes back bit for bit; every
# value is within half a step of the grid at its magnitude; and an exact
# midpoint between two neighbours rounds to the even mantissa.
def pin_e4m3_quantizer(quantize, decode, seed=34):
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((6, 512)) * np.array([1e-3, 0.5, 1.0, 3.0, 100.0, 1e4])[:, None]
    codes, scale = quantize(rows)
    back = decode(codes) * scale.astype(np.float64)[:, None]
    for r in range(rows.shape[0]):
        k = np.argmax(np.abs(rows[r]))
        assert abs(decode(codes[r, k:k + 1])[0]) == 448.0, "row maximum must map to 448"
        y = rows[r] / float(scale[r])
        # grid step at |y|: 2^(e-3) for normals (e = floor(log2|y|)), 2^-9 below 2^-6
        e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
        step = 2.0 ** (e - 3)
        err = np.abs(back[r] / float(scale[r]) - y)
        assert np.all(err <= step / 2 * (1 + 1e-12)), "quantisation error above half a step"
    exact = decode(rng.integers(0, 0x7F, size=(3, 512)).astype(np.uint8))
    exact[:, 0] = 448.0                    # fixes amax, so scale = 2^k exactly
    exact *= 2.0 ** np.array([-3, 0, 5])[:, None]
    c2, s2 = quantize(exact)
    assert np.array_equal(decode(c2) * s2.astype(np.float64)[:, None], exact), "exact values not kept"
    # midpoints: 1 + 1/16 lies between 1 (even mantissa 0) and 1.125 (odd);
    # 1.125 + 1/16 between 1.125 (odd) and 1.25 (even)
    row = np.zeros((1, 512))
    row[0, 0] = 448.0
    row[0, 1], row[0, 2] = 1.0625, 1.1875
    c3, s3 = quantize(row)
    assert float(s3[0]) == 1.0
    assert decode(c3[0, 1:3]).tolist() == [1.0, 1.25], "ties must go to the even mantissa"


# (q) FP8 decode against the BF16 path: when every latent value is exactly
# an E4M3 value times a power-of-two scale (so also exactly a BF16 value),
# decode over the FP8 cache equals the BF16 reference over the same rows
# written as BF16, bit for bit.
def pin_fp8_decode_matches_bf16(decode_fp8, ref_bits, seed=35):
    from workloads import bf16_round_bits
    rng = np.random.default_rng(seed)
    inp = make_inputs([70, 5, 129], s_q=2, h_q=4, seed=seed, causal=True)
    pages = inp.kv_bits.shape[0]
    codes = rng.integers(0, 0x7F, size=(pages, 64, 512)).astype(np.uint8)
    codes[rng.random(codes.shape) < 0.5] |= 0x80                     # both signs
    scales = (2.0 ** rng.integers(-8, -3, size=(pages, 64))).astype(np.float32)
    rope = inp.kv_bits[:, :, 0, 512:]
    lat = oracle.e4m3_decode(codes) * scales.astype(np.float64)[..., None]
    kv_bits = np.concatenate([bf16_round_bits(lat.astype(np.float32)), rope], axis=-1)[:, :, None, :]
    assert np.array_equal(_f64(kv_bits[..., :512])[:, :, 0], lat), "test rows not exact in BF16"
    o1, l1 = decode_fp8(inp.q_bits, codes, rope, scales, inp.block_table, inp.seqlens, inp.scale, True)
    o2, l2 = ref_bits(inp.q_bits, kv_bits, inp.block_table, inp.seqlens, inp.scale, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "FP8 decode differs from BF16 decode"


# (r) Quantiser against brute force in exact rational arithmetic: for every
# value, the code whose E4M3 value is nearest to the exact quotient
# |x| / scale (Fraction arithmetic; all 127 magnitudes tried in a plain loop;
# ties to the even code; at or above 448 saturating to 0x7E), with x's sign
# bit, and scale equal to the FP32 number nearest amax / 448. Rows mix tiny
# values (subnormal codes, negative values that round to zero), values near
# midpoints and the row maximum.
def pin_e4m3_quantizer_bruteforce(quantize, decode, seed=36):
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    rows = (rng.standard_normal((3, 512)) * np.array([1.0, 1e-3, 50.0])[:, None]).astype(np.float32)
    rows[0, :8] = [448.0, -1e-9, 1e-9, 2.0 ** -10, -(2.0 ** -10), 7.5 * 2 ** -9, 0.0, -0.0]
    codes, scale = quantize(rows)
    mags = [Fraction(float(decode(np.array([c], dtype=np.uint8))[0])) for c in range(0x7F)]
    for r in range(rows.shape[0]):
        amax = Fraction(float(np.abs(rows[r]).max()))
        s_exact = amax / 448
        # the scale is the FP32 number nearest amax / 448: no FP32 number lies
        # closer (its two FP32 neighbours are no nearer)
        s32 = float(scale[r])
        up, down = np.nextafter(np.float32(s32), np.float32(np.inf)), np.nextafter(np.float32(s32), np.float32(0))
        assert abs(Fraction(s32) - s_exact) <= abs(Fraction(float(up)) - s_exact), "scale not nearest"
        assert abs(Fraction(s32) - s_exact) <= abs(Fraction(float(down)) - s_exact), "scale not nearest"
        for d in range(0, 512, 3):
            t = abs(Fraction(float(rows[r, d]))) / Fraction(s32)
            if t >= 448:
                best = 0x7E
            else:
                dist = [abs(m - t) for m in mags]
                dmin = min(dist)
                cands = [c for c in range(0x7F) if dist[c] == dmin]
                best = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
            want = best | (0x80 if math.copysign(1.0, float(rows[r, d])) < 0 else 0)
            assert codes[r, d] == want, f"row {r} col {d}: t={float(t)!r} code 0x{codes[r, d]:02x} want 0x{want:02x}"


# (v) The quotient is exact, not an FP32 quotient. With amax = 11 the scale
# is fl32(11/448), and for x = 1.03125 (and its multiples by powers of two)
# the FP32 quotient fl32(x / scale) is exactly 42, the midpoint between the
# grid values 40 (code 0x62, even) and 44 (code 0x63). The exact quotient
# lies just above 42, so the nearest value is 44: an FP32 quotient followed
# by ties-to-even would give 40 instead. A second row checks the mirror case
# (an exact quotient just below an FP32 midpoint whose even neighbour is
# above) found by a plain search over BF16 values, and a third a value whose
# exact quotient is itself a midpoint (ties to even).
def pin_e4m3_exact_quotient(quantize, decode):
    from fractions import Fraction
    row = np.zeros((1, 512), dtype=np.float32)
    row[0, 0] = 11.0
    xs = [1.03125 * 2.0 ** k for k in range(-4, 4)]
    row[0, 1:1 + len(xs)] = xs
    codes, scale = quantize(row)
    s32 = np.float32(11.0) / np.float32(448.0)
    assert scale[0] == s32
    grid = [float(decode(np.array([c], dtype=np.uint8))[0]) for c in range(0x7F)]
    mids = {(grid[k] + grid[k + 1]) / 2: k for k in range(0x7E)}
    for j, x in enumerate(xs, start=1):
        y32 = float(np.float32(np.float32(x) / s32))
        assert y32 in mids and mids[y32] % 2 == 0, f"x={x}: FP32 quotient {y32} is not an even-below midpoint"
        assert Fraction(x) / Fraction(float(s32)) > Fraction(y32), "exact quotient above the FP32 one"
        val = float(decode(codes[0, j:j + 1])[0])
        assert val == grid[mids[y32] + 1], f"x={x}: code 0x{codes[0, j]:02x} ({val}), nearest is {grid[mids[y32] + 1]}"
    assert codes[0, 5] == 0x63 and float(decode(codes[0, 5:6])[0]) == 44.0
    # mirror case: search BF16 values x <= amax whose FP32 quotient is a
    # midpoint k with k odd (its even neighbour is the upper one) while the
    # exact quotient lies below: the nearest value is then the lower, odd code
    found = None
    xs_all = (np.arange(0x0080, 0x4200, dtype=np.uint32) << 16).view(np.float32)   # BF16 2^-126 .. 2^5
    mid_vals = np.array(sorted(mids), dtype=np.float64)
    for amax in (3.0, 5.0, 6.5, 9.0, 11.0, 13.0):
        s = np.float32(amax) / np.float32(448.0)
        xs_a = xs_all[xs_all <= amax]
        y32s = (xs_a / s).astype(np.float32)
        for x, y32 in zip(xs_a[np.isin(y32s.astype(np.float64), mid_vals)], y32s[np.isin(y32s.astype(np.float64), mid_vals)]):
            k = mids[float(y32)]
            if k % 2 == 1 and Fraction(float(x)) / Fraction(float(s)) < Fraction(float(y32)):
                found = (amax, float(x), k)
                break
        if found:
            break
    assert found is not None, "no mirror case in the searched range"
    amax, x, k = found
    row2 = np.zeros((1, 512), dtype=np.float32)
    row2[0, 0], row2[0, 1] = amax, x
    c2, _ = quantize(row2)
    assert c2[0, 1] == k, f"amax={amax} x={x}: code 0x{c2[0, 1]:02x}, nearest is 0x{k:02x}"
    # an exact midpoint: amax = 448 gives scale 1, and 42 = (40 + 44) / 2
    row3 = np.zeros((1, 512), dtype=np.float32)
    row3[0, 0], row3[0, 1], row3[0, 2] = 448.0, 42.0, -46.0
    c3, s3 = quantize(row3)
    assert float(s3[0]) == 1.0 and c3[0, 1] == 0x62 and c3[0, 2] == 0xE4, "exact midpoints go to the even code"


# (s) FP8 append from the physical side, as (k): every page row the placement
# rule sends a token to holds that token's quantised latent bytes, its scale
# and its rotary bits; every other row is unchanged; tokens without a page
# are counted.
def pin_append_fp8_physical_view(append_fp8, quantize, seed=37):
    for inp in _append_cases(seed):
        pages = inp.kv_bits.shape[0]
        rng = np.random.default_rng(seed)
        codes0 = rng.integers(0, 256, size=(pages, PAGE, 512)).astype(np.uint8)
        rope0 = inp.kv_bits[:, :, 0, 512:].copy()
        sc0 = rng.random((pages, PAGE)).astype(np.float32)
        c1, r1, s1, skipped = append_fp8(codes0, rope0, sc0, inp.new_bits, inp.block_table, inp.seqlens)
        ec, er, es = codes0.copy(), rope0.copy(), sc0.copy()
        s_new = inp.new_bits.shape[1]
        written = 0
        for b in range(inp.block_table.shape[0]):
            first_new = int(inp.seqlens[b]) - s_new
            for logical in range(inp.block_table.shape[1]):
                page = int(inp.block_table[b, logical])
                if not 0 <= page < pages:
                    continue
                for slot in range(PAGE):
                    i = logical * PAGE + slot - first_new
                    if 0 <= i < s_new:
                        x = bf16_bits_to_f32(inp.new_bits[b, i, :512])[None]
                        q, sq = quantize(x)
                        ec[page, slot], es[page, slot] = q[0], sq[0]
                        er[page, slot] = inp.new_bits[b, i, 512:]
                        written += 1
        placed = sum(min(int(n), s_new) for n in inp.seqlens)
        assert np.array_equal(c1, ec) and np.array_equal(r1, er), "latent or rotary rows wrong"
        assert np.array_equal(s1.view(np.uint32), es.view(np.uint32)), "scales wrong"
        assert skipped == placed - written


# (t) MHA decode against brute force: pure-Python fsum loops on tiny shapes,
# grouped heads, causal and not, a sequence shorter than s_q.
def pin_mha_bruteforce(mha, seed=38):
    from workloads import make_mha_inputs
    for causal in (False, True):
        inp = make_mha_inputs([3, 70, 1], 2, 4, 2, 16, seed + causal, causal=causal)
        o, l = mha(inp.q_bits, inp.k_bits, inp.v_bits, inp.block_table, inp.seqlens, inp.scale, causal)
        f = lambda bits: bf16_bits_to_f32(bits).astype(np.float64)
        ob, lb = oracle.mha_decode_bruteforce(f(inp.q_bits), f(inp.k_bits), f(inp.v_bits), inp.block_table,
                                              inp.seqlens, float(np.float32(inp.scale)), causal)
        assert np.abs(o - ob).max() < 1e-12, "MHA output vs brute force"
        fin = np.isfinite(lb)
        assert np.array_equal(fin, np.isfinite(l)) and np.abs(l[fin] - lb[fin]).max() < 1e-12


# (u) Grouping: giving every query head its own copy of its group's KV head
# (H_kv = H_q) leaves every output unchanged; a single cached token returns
# its value vector; relabelling physical pages changes nothing.
def pin_mha_grouping_and_invariants(mha, seed=39):
    import dataclasses
    from workloads import make_mha_inputs, permute_pages
    inp = make_mha_inputs([37, 100, 64, 129], 1, 8, 2, 32, seed)
    o1, l1 = mha(inp.q_bits, inp.k_bits, inp.v_bits, inp.block_table, inp.seqlens, inp.scale, False)
    k_full = np.repeat(inp.k_bits, 4, axis=2)
    v_full = np.repeat(inp.v_bits, 4, axis=2)
    o2, l2 = mha(inp.q_bits, k_full, v_full, inp.block_table, inp.seqlens, inp.scale, False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "grouping"
    one = make_mha_inputs([1, 1], 1, 4, 2, 32, seed + 1)
    o3, _ = mha(one.q_bits, one.k_bits, one.v_bits, one.block_table, one.seqlens, one.scale, False)
    for b in range(2):
        page = one.block_table[b, 0]
        for h in range(4):
            assert np.array_equal(o3[b, 0, h], bf16_bits_to_f32(one.v_bits[page, 0, h // 2]).astype(np.float64))
    # page relabelling: permute_pages moves MlaInputs' kv_bits; move K and V alike
    rng = np.random.default_rng(seed + 2)
    pi = rng.permutation(inp.k_bits.shape[0])
    k_p = np.empty_like(inp.k_bits)
    v_p = np.empty_like(inp.v_bits)
    k_p[pi], v_p[pi] = inp.k_bits, inp.v_bits
    table = np.where(inp.block_table >= 0, pi[np.maximum(inp.block_table, 0)], inp.block_table).astype(np.int32)
    o4, l4 = mha(inp.q_bits, k_p, v_p, table, inp.seqlens, inp.scale, False)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4), "page relabelling"
