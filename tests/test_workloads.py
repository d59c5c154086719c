"""Input generator checks (CPU): determinism, storage rounding, e4m3 codes, enlarged keys."""

import numpy as np
import torch

import workloads


def test_workload_table():
    w = workloads.WORKLOADS
    assert [x.number for x in w.values()] == [1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 14]
    assert w["onehead_32k"].shape() == (1, 1, 32768, 128) and w["onehead_32k"].backward
    assert w["fp8bwd_8k"].fp8 and w["fp8bwd_8k"].backward
    assert w["d96_4k"].shape() == (4, 32, 4096, 96)
    assert w["d256_4k"].shape() == (4, 16, 4096, 256) and w["d256_4k"].causal
    assert w["d256_4k"].fwd_flops() == w["causal_4k"].fwd_flops()
    assert w["fp8_d256_8k"].fwd_flops() == w["fp8_8k"].fwd_flops() and w["fp8_d256_8k"].fp8
    assert w["causal_4k"].shape() == (4, 32, 4096, 128) and w["causal_4k"].causal
    # forward 4·B·H·N²·d halved when causal; backward 2.5× forward
    assert w["causal_4k"].fwd_flops() == 4 * 4 * 32 * 4096 ** 2 * 128 / 2
    assert w["causal_4k"].bwd_flops() == 2.5 * w["causal_4k"].fwd_flops()
    assert abs(w["causal_4k"].fwd_flops() + w["causal_4k"].bwd_flops() - 1924.1e9) < 0.1e9


def test_inputs_are_deterministic_and_distinct():
    a = workloads.make_inputs("d64_2k", B=1, H=2, N=64)
    b = workloads.make_inputs("d64_2k", B=1, H=2, N=64)
    for key in ("q", "k", "v", "do"):
        assert a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["q"], a["k"])
    assert not torch.equal(a["v"], a["do"])


def test_decode_workloads():
    w = workloads.DECODE_WORKLOADS
    assert [x.number for x in w.values()] == [6, 7]
    assert w["decode_32k"].q_shape() == (4, 32, 1, 128)
    assert w["specdec_32k"].kv_shape() == (4, 32, 32768, 128)
    assert w["decode_32k"].kv_bytes() == 2 * 4 * 32 * 32768 * 128 * 2
    a = workloads.make_decode_inputs("specdec_32k", B=1, H=2, Nk=70)
    b = workloads.make_decode_inputs("specdec_32k", B=1, H=2, Nk=70)
    assert a["q"].shape == (1, 2, 8, 128) and a["k"].shape == (1, 2, 70, 128)
    for key in ("q", "k", "v"):
        assert a[key].dtype == torch.bfloat16 and torch.equal(a[key], b[key])
    assert not torch.equal(a["k"], a["v"])


def _bf16_rne_bits(x):
    """Independent float32 → bfloat16 round-to-nearest-even on the bit pattern (finite inputs)."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounding = 0x7FFF + ((u >> 16) & 1)
    return ((u + rounding) >> 16).astype(np.uint16)


def test_bf16_rounding_matches_bit_reference():
    g = torch.Generator().manual_seed(7)
    x = torch.randn(1_000_000, generator=g) * torch.exp(torch.randn(1_000_000, generator=g) * 4)
    ours = workloads.to_bf16(x).view(torch.int16).numpy().view(np.uint16)
    ref = _bf16_rne_bits(x.numpy())
    assert np.array_equal(ours, ref)
    # exact ties go to even
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    got = workloads.to_bf16(torch.from_numpy(ties)).float().numpy()
    assert got[0] == 1.0 and got[1] == 1.0 + 2.0 ** -6


def _e4m3fn_value(code):
    """OCP e4m3fn decoding written from the format: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    exponent 0 is subnormal; S.1111.111 is NaN; there are no infinities."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_e4m3_table_exhaustive_and_round_trip():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        ref = _e4m3fn_value(c)
        if np.isnan(ref):
            assert np.isnan(vals[c])
            continue
        assert vals[c] == ref, c
        back = torch.tensor([ref], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
        if ref == 0.0:
            assert int(back) in (0x00, 0x80)
        else:
            assert int(back) == c
    assert np.nanmax(np.abs(vals)) == 448.0


def test_e4m3_quantiser():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4, 2, 64, 128, generator=g)
    x8, s = workloads.quantize_e4m3(x)
    assert x8.dtype == torch.float8_e4m3fn
    assert abs(s - float(x.abs().max()) / 448.0) <= 1e-7 * s
    deq = workloads.dequantized64(x8, s)
    assert torch.isfinite(deq).all()
    assert float(deq.abs().max()) <= 448.0 * s * (1 + 1e-7)
    # relative rounding error of e4m3 is at most 2^-4 for normal values; subnormal step 2^-9 · s
    err = (deq - x.double()).abs()
    bound = torch.maximum(x.double().abs() * 2.0 ** -4, torch.full_like(err, 2.0 ** -10 * s))
    assert bool((err <= bound * (1 + 1e-9)).all())
    # the clamp keeps values just past 448 finite
    y8, _ = workloads.quantize_e4m3(torch.tensor([1.0, -1.0, 0.5]))
    assert torch.isfinite(y8.to(torch.float32)).all()


def test_enlarged_keys():
    w = workloads.WORKLOADS["long_16k"]
    inp = workloads.make_inputs("long_16k", B=1, H=2, N=3000)
    plain = workloads.to_bf16(workloads.randn_f32((1, 2, 3000, 128), 1000 * w.number + 1))
    k = inp["k"]
    ratio = k.float() / plain.float()
    changed = (k != plain).any(dim=-1)
    for h in range(2):
        rows = torch.nonzero(changed[0, h]).flatten().tolist()
        # one row per 1024-key block (3 blocks for N = 3000), each multiplied by exactly 8
        assert len(rows) == 3
        assert [r // 1024 for r in rows] == [0, 1, 2]
        for r in rows:
            nz = plain[0, h, r] != 0
            assert torch.all(ratio[0, h, r][nz] == 8.0)
