"""The C ABI on the host (no GPU): the library loads, exports every entry
point the header declares, and rejects bad arguments with the documented
status before making any HIP call."""

import ctypes
import os
import re

import pytest

from mla_paged_kv_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, INVALID, UNSUPPORTED, MISALIGNED, TOO_SMALL, HIP = range(6)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_two_calls():
    names = declared_functions()
    assert "mla_get_split_metadata" in names and "mla_decode_fwd" in names
    assert "mla_kv_append" in names


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libmla_decode.so"
        assert name in _lib.SIGNATURES, f"{name} has no binding signature"


def test_status_strings():
    lib = _lib.lib()
    for code in range(7):
        assert lib.mla_status_string(code).decode().startswith(_lib.STATUS_NAMES[code])
    assert lib.mla_abi_version() >> 16 == 1


def test_size_queries():
    lib = _lib.lib()
    assert lib.mla_metadata_bytes(0, 16, 1, 64) == 0          # batch < 1
    assert lib.mla_metadata_bytes(4, 0, 1, 64) == 0           # h_q < 1
    assert lib.mla_metadata_bytes(4, 512, 4, 64) == 0         # M > MLA_MAX_ROWS
    assert lib.mla_metadata_bytes(4, 16, 1, 64) == 4 * (16 + 8 * 64 + 4 * 4 + 1 * 4)
    assert lib.mla_metadata_bytes(4, 16, 1, 60) == 4 * (16 + 8 * 64 + 4 * 4 + 1 * 4)  # rounded to 8
    ws = lib.mla_workspace_bytes(4, 16, 1, 64)
    assert ws >= 2 * 64 * 16 * 512 * 4


FAKE = 0x10000  # aligned, never dereferenced: validation fails first


def _decode(**kw):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, maxb=4, seqlens=FAKE, batch=2, s_q=1, h_q=16,
                pages=8, scale=1 / 24, causal=0, meta=FAKE, nparts=64, ws=FAKE,
                ws_bytes=1 << 30, out=FAKE, lse=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_decode_fwd(
        args["q"], args["kv"], args["bt"], args["maxb"], args["seqlens"], args["batch"],
        args["s_q"], args["h_q"], args["pages"], ctypes.c_float(args["scale"]), args["causal"],
        args["meta"], args["nparts"], args["ws"], args["ws_bytes"], args["out"], args["lse"],
        args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kv=None), INVALID), (dict(bt=None), INVALID),
    (dict(seqlens=None), INVALID), (dict(ws=None), INVALID), (dict(out=None), INVALID),
    (dict(lse=None), INVALID), (dict(batch=0), INVALID), (dict(s_q=0), INVALID),
    (dict(h_q=0), INVALID), (dict(maxb=0), INVALID), (dict(pages=0), INVALID),
    (dict(causal=2), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(nparts=70000), INVALID),
    # the contract is scale > 0: the kernels scale the raw row maximum, which
    # is the maximum of the scaled scores only for a positive scale
    (dict(scale=-1.0), INVALID), (dict(scale=-0.0), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=-float("inf")), INVALID),
    (dict(h_q=128, s_q=16), UNSUPPORTED),
    (dict(q=FAKE + 8), MISALIGNED), (dict(kv=FAKE + 4), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED),
    (dict(ws=FAKE + 8), MISALIGNED), (dict(bt=FAKE + 2), MISALIGNED), (dict(lse=FAKE + 1), MISALIGNED),
    (dict(seqlens=FAKE + 3), MISALIGNED), (dict(meta=FAKE + 2), MISALIGNED),
    (dict(ws_bytes=1024), TOO_SMALL),
])
def test_decode_argument_checks(kw, status):
    assert _decode(**kw) == status


def test_metadata_argument_checks():
    lib = _lib.lib()
    assert lib.mla_get_split_metadata(None, 2, 16, 1, 64, FAKE, 1 << 20, None) == INVALID
    assert lib.mla_get_split_metadata(FAKE, 0, 16, 1, 64, FAKE, 1 << 20, None) == INVALID
    assert lib.mla_get_split_metadata(FAKE, 2, 16, 1, 64, FAKE + 2, 1 << 20, None) == MISALIGNED
    assert lib.mla_get_split_metadata(FAKE, 2, 1024, 2, 64, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.mla_get_split_metadata(FAKE, 2, 16, 1, 64, FAKE, 16, None) == TOO_SMALL


def test_host_metadata_rejects_negative_lengths():
    import numpy as np
    sl = np.array([5, -1], dtype=np.int32)
    meta = np.zeros(4096, dtype=np.int32)
    st = _lib.lib().mla_get_split_metadata_host(sl.ctypes.data, 2, 16, 1, 8, meta.ctypes.data, meta.nbytes)
    assert st == INVALID


def test_timing_record_is_empty_without_calls():
    lib = _lib.lib()
    d, c, n = ctypes.c_double(-1), ctypes.c_double(-1), ctypes.c_int(-1)
    assert lib.mla_timing_enable(1) == OK
    assert lib.mla_timing_collect(ctypes.byref(d), ctypes.byref(c), ctypes.byref(n)) == OK
    assert (d.value, c.value, n.value) == (0.0, 0.0, 0)
    assert lib.mla_timing_collect(None, None, None) == OK
    assert lib.mla_timing_enable(0) == OK


def _append(**kw):
    args = dict(new=FAKE, batch=2, s_new=3, seqlens=FAKE, bt=FAKE, maxb=4, kv=FAKE, pages=8,
                skipped=None, stream=None)
    args.update(kw)
    return _lib.lib().mla_kv_append(args["new"], args["batch"], args["s_new"], args["seqlens"],
                                    args["bt"], args["maxb"], args["kv"], args["pages"],
                                    args["skipped"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(new=None), INVALID), (dict(seqlens=None), INVALID), (dict(bt=None), INVALID),
    (dict(kv=None), INVALID), (dict(batch=0), INVALID), (dict(s_new=0), INVALID),
    (dict(maxb=0), INVALID), (dict(pages=0), INVALID),
    (dict(batch=1 << 16, s_new=1 << 15), UNSUPPORTED),
    (dict(new=FAKE + 8), MISALIGNED), (dict(kv=FAKE + 2), MISALIGNED), (dict(bt=FAKE + 2), MISALIGNED),
    (dict(seqlens=FAKE + 1), MISALIGNED), (dict(skipped=FAKE + 2), MISALIGNED),
])
def test_append_argument_checks(kw, status):
    assert _append(**kw) == status


def _check_inputs(**kw):
    args = dict(bt=FAKE, maxb=4, seqlens=FAKE, batch=2, pages=8, out=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_check_decode_inputs(args["bt"], args["maxb"], args["seqlens"], args["batch"],
                                              args["pages"], args["out"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), INVALID), (dict(seqlens=None), INVALID), (dict(out=None), INVALID),
    (dict(batch=0), INVALID), (dict(maxb=0), INVALID), (dict(pages=0), INVALID),
    (dict(batch=1 << 16, maxb=1 << 16), UNSUPPORTED),
    (dict(bt=FAKE + 2), MISALIGNED), (dict(seqlens=FAKE + 1), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED),
])
def test_check_decode_inputs_argument_checks(kw, status):
    """Rejected on the host, before any HIP call."""
    assert _check_inputs(**kw) == status


def _absorb_q(**kw):
    args = dict(qn=FAKE, qr=FAKE, w=FAKE, tokens=4, h=2, dn=128, out=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_absorb_q(args["qn"], args["qr"], args["w"], args["tokens"], args["h"], args["dn"],
                                   args["out"], args["stream"])


def _absorb_o(**kw):
    args = dict(o=FAKE, w=FAKE, tokens=4, h=2, dv=128, out=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_absorb_o(args["o"], args["w"], args["tokens"], args["h"], args["dv"], args["out"],
                                   args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(qn=None), INVALID), (dict(qr=None), INVALID), (dict(w=None), INVALID), (dict(out=None), INVALID),
    (dict(tokens=0), INVALID), (dict(h=0), INVALID), (dict(dn=16), INVALID), (dict(dn=100), INVALID),
    (dict(dn=544), INVALID), (dict(tokens=1 << 20, h=4096), UNSUPPORTED),
    (dict(qn=FAKE + 2), MISALIGNED), (dict(qr=FAKE + 8), MISALIGNED), (dict(w=FAKE + 4), MISALIGNED),
    (dict(out=FAKE + 8), MISALIGNED),
])
def test_absorb_q_argument_checks(kw, status):
    assert _absorb_q(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), INVALID), (dict(w=None), INVALID), (dict(out=None), INVALID), (dict(tokens=0), INVALID),
    (dict(h=0), INVALID), (dict(dv=0), INVALID), (dict(dv=48), INVALID), (dict(dv=1024), INVALID),
    (dict(tokens=1 << 20, h=4096), UNSUPPORTED),
    (dict(o=FAKE + 8), MISALIGNED), (dict(w=FAKE + 2), MISALIGNED), (dict(out=FAKE + 4), MISALIGNED),
])
def test_absorb_o_argument_checks(kw, status):
    assert _absorb_o(**kw) == status


def _decode_fp8(**kw):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, maxb=4, seqlens=FAKE, batch=2, s_q=1, h_q=16,
                pages=8, scale=1 / 24, causal=0, meta=FAKE, nparts=64, ws=FAKE,
                ws_bytes=1 << 30, out=FAKE, lse=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_decode_fwd_fp8(
        args["q"], args["kv"], args["bt"], args["maxb"], args["seqlens"], args["batch"],
        args["s_q"], args["h_q"], args["pages"], ctypes.c_float(args["scale"]), args["causal"],
        args["meta"], args["nparts"], args["ws"], args["ws_bytes"], args["out"], args["lse"],
        args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(kv=None), INVALID), (dict(q=None), INVALID), (dict(batch=0), INVALID), (dict(causal=3), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=-0.0), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(h_q=128, s_q=16), UNSUPPORTED),
    (dict(kv=FAKE + 4), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED), (dict(ws_bytes=1024), TOO_SMALL),
])
def test_decode_fp8_argument_checks(kw, status):
    assert _decode_fp8(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(new=None), INVALID), (dict(kv=None), INVALID), (dict(s_new=0), INVALID), (dict(pages=0), INVALID),
    (dict(batch=1 << 16, s_new=1 << 15), UNSUPPORTED), (dict(kv=FAKE + 8), MISALIGNED),
    (dict(skipped=FAKE + 1), MISALIGNED),
])
def test_append_fp8_argument_checks(kw, status):
    args = dict(new=FAKE, batch=2, s_new=3, seqlens=FAKE, bt=FAKE, maxb=4, kv=FAKE, pages=8,
                skipped=None, stream=None)
    args.update(kw)
    assert _lib.lib().mla_kv_append_fp8(args["new"], args["batch"], args["s_new"], args["seqlens"], args["bt"],
                                        args["maxb"], args["kv"], args["pages"], args["skipped"],
                                        args["stream"]) == status


def test_fp8_metadata_argument_checks():
    lib = _lib.lib()
    assert lib.mla_get_split_metadata_fp8(None, 2, 16, 1, 64, FAKE, 1 << 20, None) == INVALID
    assert lib.mla_get_split_metadata_fp8(FAKE, 2, 128, 16, 64, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.mla_get_split_metadata_fp8(FAKE, 2, 16, 1, 64, FAKE, 16, None) == TOO_SMALL


def test_size_queries_cover_the_fp8_plan():
    # the FP8 plan of 128 and 256 rows (64-row blocks: R = 2 and 4); one
    # buffer must fit it, also for large batches
    lib = _lib.lib()
    for batch in (1, 64, 4096):
        for s_q, r in ((1, 2), (2, 4)):
            m = lib.mla_metadata_bytes(batch, 128, s_q, 64)
            w = lib.mla_workspace_bytes(batch, 128, s_q, 64)
            meta = 4 * (16 + 8 * 64 + 4 * batch + r * batch)      # P = 64
            assert m >= meta and w > 0
    # by default the BF16 plan of 32 rows has two 16-row blocks (R = 2), the
    # FP8 one a 32-row score/value block (R = 1, per-segment cost 3); under
    # the score/value override both take 32-row blocks and share the plan
    lens = [300, 70, 129, 5000]
    assert _host_plan(lens, 32, 1, 64)[8] == 2
    assert _check_meta(_host_plan(lens, 32, 1, 64), 4, 32, 1, 64, fp8=1) == INVALID
    try:
        assert lib.mla_set_plan_override(1, -1) == OK
        assert _host_plan(lens, 32, 1, 64)[3] == 3
        assert _check_meta(_host_plan(lens, 32, 1, 64), 4, 32, 1, 64, fp8=1) == OK
    finally:
        lib.mla_set_plan_override(-1, -1)


def _mha(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxb=4, seqlens=FAKE, batch=2, s_q=1, h_q=16, h_kv=8,
                pages=8, scale=1 / 24, causal=0, out=FAKE, lse=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_mha_decode_fwd(
        args["q"], args["k"], args["v"], args["bt"], args["maxb"], args["seqlens"], args["batch"],
        args["s_q"], args["h_q"], args["h_kv"], args["pages"], ctypes.c_float(args["scale"]),
        args["causal"], args["out"], args["lse"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(h_kv=0), INVALID),
    (dict(h_q=12, h_kv=8), INVALID), (dict(causal=2), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=-0.0), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(h_q=64, h_kv=2), UNSUPPORTED), (dict(q=FAKE + 8), MISALIGNED), (dict(out=FAKE + 4), MISALIGNED),
])
def test_mha_argument_checks(kw, status):
    assert _mha(**kw) == status


def _host_plan(seqlens, h_q, s_q, parts):
    import numpy as np
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    lib = _lib.lib()
    nbytes = lib.mla_metadata_bytes(len(sl), h_q, s_q, parts)
    meta = np.zeros(nbytes // 4, dtype=np.int32)
    assert lib.mla_get_split_metadata_host(sl.ctypes.data, len(sl), h_q, s_q, parts, meta.ctypes.data,
                                           meta.nbytes) == OK
    return meta


def _check_meta(meta, batch, h_q, s_q, parts, fp8=0, nbytes=None):
    return _lib.lib().mla_check_metadata_host(meta.ctypes.data, meta.nbytes if nbytes is None else nbytes,
                                              batch, h_q, s_q, parts, fp8)


def test_plan_header_check_on_host_plans():
    """The header test the decode kernels run before using a plan, through
    the host copy of the plan builder's output: a plan matches the call it
    was built for and no call that would read it at other offsets."""
    lens = [300, 70, 129, 5000]
    for h_q, s_q, parts in [(16, 1, 64), (64, 1, 64), (128, 2, 32), (16, 3, 8)]:
        meta = _host_plan(lens, h_q, s_q, parts)
        assert _check_meta(meta, 4, h_q, s_q, parts) == OK
        assert _check_meta(meta, 4, h_q, s_q, parts * 2) == INVALID      # another partition count
        assert _check_meta(meta, 3, h_q, s_q, parts) == INVALID          # another batch
        assert _check_meta(meta, 4, h_q * 2, s_q, parts) == INVALID      # other row blocks
        bad = meta.copy()
        bad[0] ^= 1
        assert _check_meta(bad, 4, h_q, s_q, parts) == INVALID           # not a plan
        assert _check_meta(meta, 4, h_q, s_q, parts, nbytes=60) == TOO_SMALL
    # by default the BF16 and FP8 calls cut 16 rows, and 64 rows and more,
    # alike (one 16-row block; 64-row blocks) and share the plan
    assert _check_meta(_host_plan(lens, 64, 1, 64), 4, 64, 1, 64, fp8=1) == OK
    assert _check_meta(_host_plan(lens, 128, 2, 64), 4, 128, 2, 64, fp8=1) == OK
    assert _check_meta(_host_plan(lens, 16, 1, 64), 4, 16, 1, 64, fp8=1) == OK
    assert _lib.lib().mla_check_metadata_host(None, 1024, 4, 16, 1, 64, 0) == INVALID
    assert _check_meta(_host_plan(lens, 16, 1, 64), 4, 16, 1, 64, fp8=2) == INVALID
    assert _check_meta(_host_plan(lens, 16, 1, 64), 4, 512, 4, 64) == UNSUPPORTED


def test_plan_override_is_checked_and_shapes_the_plan():
    lib = _lib.lib()
    assert lib.mla_set_plan_override(3, -1) == INVALID
    assert lib.mla_set_plan_override(-1, -2) == INVALID
    lens = [300, 70, 129, 5000]
    try:
        assert lib.mla_set_plan_override(1, -1) == OK          # 32-row score/value blocks at 32 rows: R = 1
        ws_plan = _host_plan(lens, 32, 1, 64)
        assert ws_plan[8] == 1 and ws_plan[3] == 3
        assert lib.mla_set_plan_override(0, -1) == OK          # 16-row blocks at 64 rows: R = 4
        r16_plan = _host_plan(lens, 64, 1, 64)
        assert r16_plan[8] == 4
        assert lib.mla_set_plan_override(2, 1) == OK           # 128-row fused-wave blocks at 64 rows: R = 1
        fw_plan = _host_plan(lens, 64, 1, 64)
        assert fw_plan[8] == 1 and fw_plan[3] == 9
        # a plan built under one setting does not match a call under the default
        assert lib.mla_set_plan_override(-1, -1) == OK
        assert _check_meta(ws_plan, 4, 32, 1, 64) == INVALID
        assert _check_meta(r16_plan, 4, 64, 1, 64) == INVALID
        assert _check_meta(fw_plan, 4, 64, 1, 64) == INVALID
    finally:
        lib.mla_set_plan_override(-1, -1)


def test_default_plan_row_blocks():
    """Row blocks of the default plans: 16 rows below 64 rows per sequence,
    64 from there (header word 8 is R, word 3 the per-segment cost
    1 + rows/16)."""
    lens = [300, 70, 129, 5000]
    for h_q, s_q, r, cseg in [(16, 1, 1, 2), (32, 1, 2, 2), (64, 1, 1, 5), (64, 2, 2, 5), (128, 1, 2, 5),
                              (128, 2, 4, 5), (128, 8, 16, 5)]:
        plan = _host_plan(lens, h_q, s_q, 64)
        assert (plan[8], plan[3]) == (r, cseg), (h_q, s_q, plan[:9])


def _noalloc(**kw):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, maxb=4, seqlens=FAKE, batch=2, s_q=1, h_q=16,
                pages=8, scale=1 / 24, causal=0, meta=FAKE, nparts=64, out=FAKE, lse=FAKE, stream=None)
    args.update(kw)
    return _lib.lib().mla_decode_fwd_noalloc(
        args["q"], args["kv"], args["bt"], args["maxb"], args["seqlens"], args["batch"],
        args["s_q"], args["h_q"], args["pages"], ctypes.c_float(args["scale"]), args["causal"],
        args["meta"], args["nparts"], args["out"], args["lse"], args["stream"])


SCRATCH_LIMIT = 6


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kv=None), INVALID), (dict(out=None), INVALID), (dict(lse=None), INVALID),
    (dict(batch=0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=0.0), INVALID), (dict(causal=2), INVALID),
    (dict(h_q=128, s_q=16), UNSUPPORTED), (dict(q=FAKE + 8), MISALIGNED), (dict(meta=FAKE + 2), MISALIGNED),
    # 4096 partitions of 1024 rows: 32 GiB of partials, far past the scratch
    (dict(h_q=128, s_q=8, nparts=4096), SCRATCH_LIMIT),
    (dict(batch=9000, h_q=128, s_q=8, nparts=512, meta=None), SCRATCH_LIMIT),
])
def test_noalloc_argument_checks(kw, status):
    """Checked on the host before any HIP call, the scratch limit included."""
    assert _noalloc(**kw) == status
