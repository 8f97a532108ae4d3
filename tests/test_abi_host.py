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
    for code in range(6):
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
    (dict(h_q=128), UNSUPPORTED), (dict(h_q=16, s_q=8), UNSUPPORTED),
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
    assert lib.mla_get_split_metadata_fp8(FAKE, 2, 128, 1, 64, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.mla_get_split_metadata_fp8(FAKE, 2, 16, 1, 64, FAKE, 16, None) == TOO_SMALL


def test_size_queries_cover_the_fp8_plan():
    # at 64 rows the BF16 plan uses the 64-row kernel, the FP8 plan the
    # 16-row one; one buffer must fit either, also for large batches
    lib = _lib.lib()
    for batch in (1, 64, 4096):
        m = lib.mla_metadata_bytes(batch, 64, 1, 64)
        w = lib.mla_workspace_bytes(batch, 64, 1, 64)
        meta16 = 4 * (16 + 8 * 64 + 4 * batch + 4 * batch)      # P = 64, R = 4
        assert m >= meta16 and w > 0
