"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them. A pin suite that still passes with a dropped term, a
wrong index or sign, or a transposed operand would not be pinning anything.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.mla_ref as R
import oracle_pins as P


def _run_all_pins():
    """Returns the names of pins that fail (AssertionError or any exception)."""
    pins = [
        ("nonabsorbed", lambda: P.pin_nonabsorbed_identity(R.mla_decode_ref_f64)),
        ("permutation", lambda: P.pin_page_permutation(R.mla_decode_ref)),
        ("single_token", lambda: P.pin_single_token(R.mla_decode_ref)),
        ("equal_scores", lambda: P.pin_equal_scores(R.mla_decode_ref_f64)),
        ("causal", lambda: P.pin_causal_reductions(R.mla_decode_ref)),
        ("combine", lambda: P.pin_combine_identity(R.attend_rows, R.lse_combine_ref)),
        ("bruteforce", lambda: P.pin_bruteforce(R.mla_decode_ref_f64)),
        ("bounds", lambda: P.pin_bounds(R.mla_decode_ref)),
        ("two_keys", lambda: P.pin_two_keys(R.mla_decode_ref_f64)),
    ]
    failed = []
    with np.errstate(all="ignore"):
        for name, fn in pins:
            try:
                fn()
            except Exception:  # noqa: BLE001 - any failure counts as caught
                failed.append(name)
    return failed


def _attend_variant(scores_fn=None, values_fn=None, lse_fn=None, weight_fn=None):
    """attend_rows with one step replaced."""
    def attend(q, k, lengths, scale):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        out = np.zeros((q.shape[0], 512))
        lse = np.full(q.shape[0], -np.inf)
        if k.shape[0] == 0:
            return out, lse
        scores = scores_fn(q, k, scale) if scores_fn else scale * (q @ k.T)
        values = values_fn(k) if values_fn else k[:, :512]
        for r in range(q.shape[0]):
            L = int(lengths[r])
            if L == 0:
                continue
            s = scores[r, :L]
            m = s.max()
            total = np.exp(s - m).sum()
            lse[r] = lse_fn(m, total) if lse_fn else m + math.log(total)
            p = weight_fn(s, m, lse[r]) if weight_fn else np.exp(s - lse[r])
            out[r] = p @ values[:L]
        return out, lse
    return attend


def _gather_variant(page_of, slot_of):
    def gather(kv, table_row, n):
        if n == 0:
            return np.zeros((0, kv.shape[-1]), dtype=kv.dtype)
        t = np.arange(n)
        return kv[np.asarray(table_row)[page_of(t)], slot_of(t), 0, :]
    return gather


MUTATIONS = {
    "gather_page_slot_swapped": ("gather_sequence_rows",
                                 _gather_variant(lambda t: t % 64, lambda t: t // 64)),
    "gather_slot_off_by_one": ("gather_sequence_rows",
                               _gather_variant(lambda t: t // 64, lambda t: (t + 1) % 64)),
    "gather_ignores_block_table": ("gather_sequence_rows",
                                   _gather_variant(lambda t: t // 64 * 0, lambda t: t % 64)),
    "rotary_term_dropped": ("attend_rows", _attend_variant(
        scores_fn=lambda q, k, sc: sc * (q[:, :512] @ k[:, :512].T))),
    "scale_missing": ("attend_rows", _attend_variant(scores_fn=lambda q, k, sc: q @ k.T)),
    "scale_squared": ("attend_rows", _attend_variant(scores_fn=lambda q, k, sc: sc * sc * (q @ k.T))),
    "values_take_rotary_part": ("attend_rows", _attend_variant(values_fn=lambda k: k[:, 64:])),
    "lse_sign": ("attend_rows", _attend_variant(lse_fn=lambda m, tot: m - math.log(tot))),
    "lse_log2": ("attend_rows", _attend_variant(lse_fn=lambda m, tot: m + math.log2(tot))),
    "weights_not_normalised": ("attend_rows", _attend_variant(weight_fn=lambda s, m, l: np.exp(s - m))),
    "causal_off_by_one": ("visible_length",
                          lambda n, s_q, i, c: n if not c else max(0, min(n, n - s_q + i))),
    "causal_reversed": ("visible_length",
                        lambda n, s_q, i, c: n if not c else max(0, min(n, n - i))),
    "causal_ignored": ("visible_length", lambda n, s_q, i, c: n),
}


def _combine_plain_average(o_parts, lse_parts):
    o_parts = np.asarray(o_parts)
    lse_parts = np.asarray(lse_parts)
    fin = np.isfinite(lse_parts)
    cnt = np.maximum(fin.sum(axis=0), 1)
    m = np.where(fin, lse_parts, -np.inf).max(axis=0)
    lse = m + np.log(np.where(fin, np.exp(lse_parts - np.where(np.isfinite(m), m, 0)), 0).sum(axis=0))
    return (o_parts * fin[..., None]).sum(axis=0) / cnt[..., None], lse


def test_unmutated_oracle_passes_every_pin():
    assert _run_all_pins() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    failed = _run_all_pins()
    assert failed, f"mutation {name} passed every pin"


def test_layout_mutation_token_head_order_is_caught(monkeypatch):
    """Rows of a sequence flattened as (head, token) instead of (token, head)."""
    real = R.mla_decode_ref_f64

    def swapped(q, kv, table, seqlens, scale, causal, seqs=None):
        q = np.asarray(q, dtype=np.float64)
        qs = np.ascontiguousarray(q.transpose(0, 2, 1, 3)).reshape(q.shape)
        return real(qs, kv, table, seqlens, scale, causal, seqs)

    monkeypatch.setattr(R, "mla_decode_ref_f64", swapped)
    assert _run_all_pins(), "token/head order swap passed every pin"


def test_combine_mutation_is_caught(monkeypatch):
    monkeypatch.setattr(R, "lse_combine_ref", _combine_plain_average)
    assert "combine" in _run_all_pins()


# ---- cache append -----------------------------------------------------------

def _append_variant(pos_fn=None, slot_fn=None, table_row_fn=None, keep_negative=False,
                    count_negative=False, wrap_width=False):
    """kv_append_ref with one step replaced."""
    def append(kv_bits, new_bits, block_table, seqlens):
        kv = np.array(kv_bits, copy=True)
        bsz, s_new, _ = new_bits.shape
        width = block_table.shape[1]
        skipped = 0
        for b in range(bsz):
            n = int(seqlens[b])
            for i in range(s_new):
                pos = pos_fn(n, s_new, i) if pos_fn else n - s_new + i
                if pos < 0 and not keep_negative:
                    if count_negative:
                        skipped += 1
                    continue
                logical = pos // 64
                row = table_row_fn(b) if table_row_fn else b
                if wrap_width:
                    page = int(block_table[row, logical % width])
                else:
                    page = int(block_table[row, logical]) if logical < width else -1
                if page < 0 or page >= kv.shape[0]:
                    skipped += 1
                    continue
                slot = slot_fn(pos, i) if slot_fn else pos % 64
                kv[page, slot, 0, :] = new_bits[b, i, :]
        return kv, skipped
    return append


APPEND_MUTATIONS = {
    "position_off_by_one": _append_variant(pos_fn=lambda n, s, i: n - s + i + 1),
    "position_from_start": _append_variant(pos_fn=lambda n, s, i: i),
    "negative_positions_written": _append_variant(keep_negative=True),
    "negative_positions_counted": _append_variant(count_negative=True),
    "slot_from_token_index": _append_variant(slot_fn=lambda pos, i: i % 64),
    "first_sequence_table_row": _append_variant(table_row_fn=lambda b: 0),
    "table_index_wraps": _append_variant(wrap_width=True),
}


def _run_append_pins(fn):
    failed = []
    for name, pin in [("physical", P.pin_append_physical_view), ("round_trip", P.pin_append_round_trip)]:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(name)
    return failed


def test_unmutated_append_passes_its_pins():
    assert _run_append_pins(oracle.kv_append_ref) == []


@pytest.mark.parametrize("name", sorted(APPEND_MUTATIONS))
def test_append_mutation_is_caught(name):
    assert _run_append_pins(APPEND_MUTATIONS[name]), f"append mutation {name} passed every pin"


# ---- absorption ----------------------------------------------------------------

def _absorb_q_variant(head_fn=None, rope_fn=None, scale=1.0):
    def absorb_q(q_nope, q_rope, w_uk):
        q_nope = np.asarray(q_nope, dtype=np.float64)
        tokens, heads, dn = q_nope.shape
        out = np.empty((tokens, heads, 576))
        for h in range(heads):
            w = w_uk[head_fn(h, heads) if head_fn else h]
            out[:, h, :512] = scale * (q_nope[:, h, :] @ w.T)
        out[:, :, 512:] = rope_fn(q_rope) if rope_fn else q_rope
        return out
    return absorb_q


def _absorb_o_variant(head_fn=None, scale=1.0, token_shift=False):
    def absorb_o(o_lat, w_uv):
        o_lat = np.asarray(o_lat, dtype=np.float64)
        tokens, heads, _ = o_lat.shape
        out = np.empty((tokens, heads, w_uv.shape[-1]))
        for h in range(heads):
            out[:, h, :] = scale * (o_lat[:, h, :] @ w_uv[head_fn(h, heads) if head_fn else h])
        if token_shift:
            out = np.roll(out, 1, axis=0)
        return out
    return absorb_o


ABSORB_MUTATIONS = {
    "q_wrong_head": (_absorb_q_variant(head_fn=lambda h, n: (h + 1) % n), None),
    "q_rope_dropped": (_absorb_q_variant(rope_fn=lambda r: np.zeros_like(r)), None),
    "q_rope_other_head": (_absorb_q_variant(rope_fn=lambda r: np.roll(r, 1, axis=1)), None),
    "q_extra_scale": (_absorb_q_variant(scale=1.0 / math.sqrt(128)), None),
    "o_wrong_head": (None, _absorb_o_variant(head_fn=lambda h, n: (h + 1) % n)),
    "o_extra_scale": (None, _absorb_o_variant(scale=0.5)),
    "o_token_order": (None, _absorb_o_variant(token_shift=True)),
}


def _run_absorb_pins(aq, ao):
    failed = []
    pins = [("end_to_end", lambda: P.pin_absorb_end_to_end(aq, ao, R.mla_decode_ref_f64)),
            ("selection", lambda: P.pin_absorb_selection(aq, ao))]
    for name, fn in pins:
        try:
            fn()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(name)
    return failed


def test_unmutated_absorb_passes_its_pins():
    assert _run_absorb_pins(oracle.absorb_q_ref, oracle.absorb_o_ref) == []


@pytest.mark.parametrize("name", sorted(ABSORB_MUTATIONS))
def test_absorb_mutation_is_caught(name):
    aq, ao = ABSORB_MUTATIONS[name]
    assert _run_absorb_pins(aq or oracle.absorb_q_ref, ao or oracle.absorb_o_ref), \
        f"absorb mutation {name} passed every pin"


# ---- FP8 cache -------------------------------------------------------------------

def _e4m3_variant(bias=7, subnormal_implicit=False, ignore_sign=False):
    def value(byte):
        sign = 1.0 if (ignore_sign or not byte & 0x80) else -1.0
        exp, man = (byte >> 3) & 0xF, byte & 0x7
        if exp == 0xF and man == 0x7:
            return math.nan
        if exp == 0 and not subnormal_implicit:
            return sign * (man / 8.0) * 2.0 ** (1 - bias)
        return sign * (1.0 + man / 8.0) * 2.0 ** (exp - bias)
    table = np.array([value(b) for b in range(256)])
    return lambda codes: table[np.asarray(codes, dtype=np.uint8)]


def _quantize_variant(ties_away=False, limit=448.0):
    def quantize(rows):
        rows = np.asarray(rows, dtype=np.float64)
        amax = np.abs(rows).max(axis=1)
        scale = np.where(amax > 0, amax / limit, 1.0).astype(np.float32)
        y = rows / scale.astype(np.float64)[:, None]
        codes = np.array([b for b in range(256) if not math.isnan(oracle.e4m3_value(b)) and b != 0x80])
        vals = np.array([oracle.e4m3_value(b) for b in codes])
        out = np.empty(y.shape, dtype=np.uint8)
        for idx, x in np.ndenumerate(y):
            d = np.abs(vals - x)
            best = np.flatnonzero(d == d.min())
            if len(best) > 1:
                best = [max(best, key=lambda k: abs(vals[k]))] if ties_away else \
                       [k for k in best if codes[k] & 1 == 0][:1]
            out[idx] = codes[best[0]]
        return out, scale
    return quantize


def _quantize_fp32_quotient(rows):
    """The quantiser with the quotient rounded to FP32 first: y = fl32(x /
    scale), then the E4M3 value nearest y, ties to even. It differs from the
    exact definition only where fl32(x / scale) lands on a midpoint that the
    exact quotient misses."""
    x = np.asarray(rows, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = (x / scale[:, None]).astype(np.float32)
    grid = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mag = np.abs(y).astype(np.float64)
    idx = np.clip(np.searchsorted(grid, mag), 1, grid.size - 1)
    lo, hi = grid[idx - 1], grid[idx]
    pick_hi = ((hi - mag) < (mag - lo)) | (((hi - mag) == (mag - lo)) & (idx % 2 == 0))
    code = np.where(mag >= 448.0, 0x7E, np.where(pick_hi, idx, idx - 1))
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8), scale


def _decode_fp8_variant(rope_scaled=False, scale_ignored=False):
    def decode(q_bits, codes, rope_bits, scales, table, seqlens, scale, causal, seqs=None):
        q = (np.asarray(q_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        s = np.ones_like(scales, dtype=np.float64) if scale_ignored else scales.astype(np.float64)
        lat = oracle.e4m3_decode(codes) * s[..., None]
        rope = (np.asarray(rope_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        rope = rope.astype(np.float64) * (s[..., None] if rope_scaled else 1.0)
        kv = np.concatenate([lat, rope], axis=-1)[:, :, None, :]
        return R.mla_decode_ref_f64(q.astype(np.float64), kv, table, seqlens, float(np.float32(scale)), causal, seqs)
    return decode


def _run_fp8_pins(decode=None, quantize=None, fp8_decode=None):
    decode = decode or oracle.e4m3_decode
    quantize = quantize or oracle.quantize_e4m3_rows
    fp8_decode = fp8_decode or oracle.mla_decode_fp8_ref
    failed = []
    pins = [("table", lambda: P.pin_e4m3_table(decode)),
            ("quantizer", lambda: P.pin_e4m3_quantizer(quantize, decode)),
            ("quantizer_bruteforce", lambda: P.pin_e4m3_quantizer_bruteforce(quantize, decode)),
            ("exact_quotient", lambda: P.pin_e4m3_exact_quotient(quantize, decode)),
            ("fp8_vs_bf16", lambda: P.pin_fp8_decode_matches_bf16(fp8_decode, R.mla_decode_ref))]
    with np.errstate(all="ignore"):
        for name, fn in pins:
            try:
                fn()
            except Exception:  # noqa: BLE001 - any failure counts as caught
                failed.append(name)
    return failed


FP8_MUTATIONS = {
    "bias_8": dict(decode=_e4m3_variant(bias=8)),
    "subnormal_as_normal": dict(decode=_e4m3_variant(subnormal_implicit=True)),
    "sign_ignored": dict(decode=_e4m3_variant(ignore_sign=True)),
    "quantize_ties_away": dict(quantize=_quantize_variant(ties_away=True)),
    "quantize_limit_240": dict(quantize=_quantize_variant(limit=240.0)),
    "quantize_fp32_quotient": dict(quantize=_quantize_fp32_quotient),
    "rope_scaled": dict(fp8_decode=_decode_fp8_variant(rope_scaled=True)),
    "scale_ignored": dict(fp8_decode=_decode_fp8_variant(scale_ignored=True)),
}


def test_unmutated_fp8_passes_its_pins():
    assert _run_fp8_pins() == []


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_fp8_mutation_is_caught(name):
    assert _run_fp8_pins(**FP8_MUTATIONS[name]), f"fp8 mutation {name} passed every pin"


# ---- MHA contrast ----------------------------------------------------------------

def _mha_variant(group_fn=None, swap_kv=False, no_scale=False, causal_shift=0):
    def mha(q_bits, k_bits, v_bits, table, seqlens, scale, causal):
        f = lambda bits: (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
            np.float32).astype(np.float64)
        q, k, v = f(q_bits), f(k_bits), f(v_bits)
        if swap_kv:
            k, v = v, k
        bsz, s_q, h_q, d = q.shape
        h_kv = k.shape[2]
        group = h_q // h_kv
        sc = 1.0 if no_scale else float(np.float32(scale))
        out = np.zeros((bsz, s_q, h_q, d))
        lse = np.full((bsz, s_q, h_q), -np.inf)
        for b in range(bsz):
            n = int(seqlens[b])
            for i in range(s_q):
                L = max(0, min(n, n - s_q + i + 1 + causal_shift)) if causal else n
                for h in range(h_q):
                    if L == 0:
                        continue
                    kv = group_fn(h, group, h_kv) if group_fn else h // group
                    t = np.arange(L)
                    pages = np.asarray(table[b])[t // 64]
                    s = sc * (k[pages, t % 64, kv] @ q[b, i, h])
                    m = s.max()
                    e = np.exp(s - m)
                    lse[b, i, h] = m + math.log(e.sum())
                    out[b, i, h] = (e / e.sum()) @ v[pages, t % 64, kv]
        return out, lse
    return mha


MHA_MUTATIONS = {
    "interleaved_groups": _mha_variant(group_fn=lambda h, g, hkv: h % hkv),
    "k_v_swapped": _mha_variant(swap_kv=True),
    "scale_missing": _mha_variant(no_scale=True),
    "causal_off_by_one": _mha_variant(causal_shift=-1),
}


def _run_mha_pins(fn):
    failed = []
    for name, pin in [("bruteforce", P.pin_mha_bruteforce), ("grouping", P.pin_mha_grouping_and_invariants)]:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(name)
    return failed


def test_unmutated_mha_passes_its_pins():
    assert _run_mha_pins(oracle.mha_decode_ref) == []


@pytest.mark.parametrize("name", sorted(MHA_MUTATIONS))
def test_mha_mutation_is_caught(name):
    assert _run_mha_pins(MHA_MUTATIONS[name]), f"MHA mutation {name} passed every pin"
