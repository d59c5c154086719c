"""The kernels' rounding of results, value by value, against the CPU's rounding.

Every bf16 result (O, dQ, dK, dV, and P before the bf16 P·V product) leaves fp32 through the device
helper ``pack_bf16x2`` (v_cvt_pk_bf16_f32), and the FP8 forward rounds P to e4m3 through
``pack_e4m3x4`` (v_cvt_pk_fp8_f32).  tests/hip/fa_probe.hip runs exactly those helpers, built with
the library's flags, over values chosen here; the reference is torch's CPU cast (round to nearest,
ties to even) and, for e4m3, ``workloads.round_e4m3`` — the rounding ``quantize_e4m3`` applies to
the inputs.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "hip", "libfa_probe.so")


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    assert os.path.exists(PROBE), "tests/hip/libfa_probe.so is not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(PROBE)
    for fn in (lib.probe_pack_bf16, lib.probe_pack_e4m3):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    return lib


def _device_bf16(lib, x):
    """x: float32 CPU tensor of even length → the device's bf16 bit patterns (int64 tensor)."""
    n = x.numel()
    assert n % 2 == 0
    xd = x.contiguous().cuda()
    out = torch.empty(n // 2, dtype=torch.int32, device="cuda")
    assert lib.probe_pack_bf16(xd.data_ptr(), out.data_ptr(), n // 2,
                               torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    w = out.cpu().to(torch.int64) & 0xFFFFFFFF
    return torch.stack([w & 0xFFFF, w >> 16], dim=1).reshape(-1)


def _device_e4m3(lib, x):
    """x: float32 CPU tensor, length a multiple of 4 → the device's e4m3 bytes (int64 tensor)."""
    n = x.numel()
    assert n % 4 == 0
    xd = x.contiguous().cuda()
    out = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    assert lib.probe_pack_e4m3(xd.data_ptr(), out.data_ptr(), n // 4,
                               torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    w = out.cpu().to(torch.int64) & 0xFFFFFFFF
    return torch.stack([(w >> (8 * i)) & 0xFF for i in range(4)], dim=1).reshape(-1)


def _bits_to_f32(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint32).view(np.float32).copy())


def test_bf16_rounding_matches_cpu_rne(probe):
    """10^6 random fp32 values over the exponents results take, plus exact ties (low half 0x8000),
    both neighbours of a tie, mantissas that carry into the next binade, bf16-exact values, signed
    zeros and the largest finite values: the device's bf16 equals torch's round-to-nearest-even
    bit for bit."""
    rng = np.random.default_rng(2026)
    n = 1_000_000
    sign = rng.integers(0, 2, n, dtype=np.uint32) << 31
    expo = rng.integers(127 - 40, 127 + 40, n, dtype=np.uint32) << 23
    mant = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    rand = sign | expo | mant
    hi = (sign | expo | (mant & 0x7FFF0000))[:200_000]
    ties = hi | 0x8000
    below, above = hi | 0x7FFF, hi | 0x8001
    carry = np.concatenate([(sign | expo | 0x007FFFFF)[:25_000], (sign | expo | 0x007F8000)[:25_000]])
    exact = hi[:50_000]
    special = np.array([0, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F0000, 0x7F7F7FFF,
                        0x00800000, 0x80800000, 0x3F800000, 0x3F808000, 0x3F818000],
                       dtype=np.uint32)
    bits = np.concatenate([rand, ties, below, above, carry, exact, special])
    if bits.size % 2:
        bits = np.append(bits, np.uint32(0x3F800000))
    x = _bits_to_f32(bits)
    got = _device_bf16(probe, x)
    want = x.to(torch.bfloat16).view(torch.int16).to(torch.int64) & 0xFFFF
    bad = torch.nonzero(got != want).reshape(-1)
    assert bad.numel() == 0, [(hex(int(bits[i])), hex(int(got[i])), hex(int(want[i])))
                              for i in bad[:8]]
    # The case that separates nearest-even from other rules occurs often: both tie directions.
    t = slice(n, n + ties.size)
    assert bool((got[t] != (torch.from_numpy(ties.astype(np.int64)) >> 16)).any())
    assert bool((got[t] == (torch.from_numpy(ties.astype(np.int64)) >> 16)).any())


def _e4m3_values():
    """All non-negative finite e4m3fn values, in increasing order (codes 0x00 .. 0x7E)."""
    return torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)


def test_e4m3_rounding_matches_quantizer(probe):
    """A sweep over the range the FP8 forward's P takes (0 to 2^8) and past it: every e4m3 value,
    every midpoint between neighbours and the fp32 numbers just below and above each midpoint,
    subnormals, and 10^6 random values; both signs.  Up to |x| = 464 (the midpoint between 448 and the
    next step, 480, which rounds to even: 448) the device's e4m3 code equals workloads.round_e4m3's,
    byte for byte.  The conversion does not saturate: past 464 it gives the NaN code (0x7F, with the
    sign).  The kernel never feeds it such values: its P is at most 2^8."""
    vals = _e4m3_values().numpy().astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    mid_bits = mids.view(np.uint32)
    near = np.concatenate([(mid_bits - 1).view(np.float32), (mid_bits + 1).view(np.float32)])
    rng = np.random.default_rng(8)
    rand = np.concatenate([rng.uniform(0, 256, 500_000), rng.uniform(0, 2 ** -6, 200_000),
                           np.exp2(rng.uniform(-12, 9, 300_000))]).astype(np.float32)
    over = np.array([448.0, 449.0, 463.99, 464.0, 465.0, 480.0, 1000.0, 3.0e38], dtype=np.float32)
    pos = np.concatenate([vals, mids, near, rand, over])
    x = np.concatenate([pos, -pos]).astype(np.float32)
    pad = (-x.size) % 4
    x = np.concatenate([x, np.zeros(pad, dtype=np.float32)])
    xt = torch.from_numpy(x)
    got = _device_e4m3(probe, xt)
    want = workloads.round_e4m3(xt).view(torch.uint8).to(torch.int64)
    inside = xt.abs() <= 464.0
    bad = torch.nonzero(inside & (got != want)).reshape(-1)
    assert bad.numel() == 0, [(float(x[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]
    nan_code = torch.where(xt < 0, 0xFF, 0x7F).to(torch.int64)
    bad = torch.nonzero(~inside & (got != nan_code)).reshape(-1)
    assert bad.numel() == 0, [(float(x[i]), hex(int(got[i]))) for i in bad[:8]]
    assert int((~inside).sum()) > 1000  # the random draws reach 512
    # Midpoints exist between every pair of neighbours, so ties to even were exercised both ways.
    assert mids.size == vals.size - 1
