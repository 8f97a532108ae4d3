"""Tile tests: the decode kernels' building blocks from mla_common.h, each
run alone on the GPU (tests/tile_probe) and checked against its plain
definition computed here: the 16x16x32 BF16 MFMA in the operand and result
lane layout the kernels assume, the transposing 16-bit LDS read, the max and
sum over a row's four lane groups, and the round-to-nearest-even BF16 output
conversion. A fault in one of these would show in the parity tests as a
wrong number somewhere; here it shows as the piece that is wrong."""

import ctypes
import os

import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tile_probe", "libtile_probe.so")


def _probe():
    import torch  # noqa: F401  (load the HIP runtime torch uses first)
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(PROBE)
    for name in ("probe_mfma16", "probe_read_tr", "probe_kgroups", "probe_pack"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _bf16_bits(x):
    """float32 -> BF16 bits, round to nearest even (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_mfma16_tile_and_lane_layout():
    import torch
    lib = _probe()
    rng = np.random.default_rng(11)
    a = _bf16_bits(rng.standard_normal((16, 32)).astype(np.float32))
    b = _bf16_bits(rng.standard_normal((32, 16)).astype(np.float32))
    c = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    assert lib.probe_mfma16(ctypes.c_void_p(_dev(a).data_ptr()), ctypes.c_void_p(_dev(b).data_ptr()),
                            ctypes.c_void_p(c.data_ptr())) == 0
    torch.cuda.synchronize()
    af, bf = _bits_to_f64(a), _bits_to_f64(b)
    ref = af @ bf
    bound = 2.0 ** -22 * (np.abs(af) @ np.abs(bf)) + 1e-30
    err = np.abs(c.cpu().numpy().astype(np.float64) - ref)
    log(f"[case] mfma16 max err / bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)


def test_transposing_lds_read():
    import torch
    lib = _probe()
    src = np.arange(256, dtype=np.uint16).reshape(16, 16) * 7 + 3   # distinct values
    dst = torch.empty((64, 4), dtype=torch.int16, device="cuda")
    assert lib.probe_read_tr(ctypes.c_void_p(_dev(src).data_ptr()), ctypes.c_void_p(dst.data_ptr())) == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    want = np.empty((64, 4), dtype=np.uint16)
    for lane in range(64):
        g, i = lane // 16, lane % 16
        want[lane] = src[4 * g:4 * g + 4, i]   # column i of the group's 4 x 16 block
    assert np.array_equal(got, want)


def test_max_and_sum_over_lane_groups():
    import torch
    lib = _probe()
    rng = np.random.default_rng(12)
    x = rng.standard_normal(64).astype(np.float32) * np.float32(1000.0)
    mx = torch.empty(64, dtype=torch.float32, device="cuda")
    sm = torch.empty(64, dtype=torch.float32, device="cuda")
    assert lib.probe_kgroups(ctypes.c_void_p(_dev(x).data_ptr()), ctypes.c_void_p(mx.data_ptr()),
                             ctypes.c_void_p(sm.data_ptr())) == 0
    torch.cuda.synchronize()
    want_max = np.empty(64, np.float32)
    want_sum = np.empty(64, np.float32)
    for lane in range(64):
        i = lane % 16
        want_max[lane] = max(x[i], x[i + 16], x[i + 32], x[i + 48])
        # the order the swaps add in: (x_i + x_{i+16}) + (x_{i+32} + x_{i+48})
        want_sum[lane] = np.float32(np.float32(x[i] + x[i + 16]) + np.float32(x[i + 32] + x[i + 48]))
    assert np.array_equal(mx.cpu().numpy(), want_max)
    assert np.array_equal(sm.cpu().numpy(), want_sum)


def test_bf16_output_rounding_is_nearest_even():
    import torch
    lib = _probe()
    rng = np.random.default_rng(13)
    base = rng.standard_normal(4096).astype(np.float32) * np.float32(3.0)
    bits = base.view(np.uint32)
    # exact ties (low 16 bits 0x8000, both parities of the kept bit), one
    # below and one above them, signed zeros, the smallest normal and huge
    # finite values (FP32 subnormals are left out: whether the conversion
    # keeps or flushes them is a mode setting, not part of this check)
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    extra = np.concatenate([ties, ties - np.uint32(1), ties + np.uint32(1),
                            np.array([0x00000000, 0x80000000, 0x00800000, 0x80800000, 0x7F7F0000, 0xFF7F0000],
                                     dtype=np.uint32)]).view(np.float32)
    x = np.concatenate([base, extra]).astype(np.float32)
    x = x[: len(x) // 4 * 4]
    x = x[np.isfinite(x) & (np.abs(x.astype(np.float64)) < 3.38e38)]   # no rounding past the BF16 range
    x = x[: len(x) // 4 * 4]
    y = torch.empty(len(x), dtype=torch.int16, device="cuda")
    assert lib.probe_pack(ctypes.c_void_p(_dev(x).data_ptr()), ctypes.c_void_p(y.data_ptr()), len(x)) == 0
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint16), _bf16_bits(x))
