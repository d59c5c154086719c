"""GPU parity of decoding against a key/value cache (fa_decode through the C ABI) with the fp64 oracle.

The queries are the last Nq positions of the sequence; the oracle is the plain definition with the
query offset Nk − Nq (oracle.attention_head_fwd64(..., q_offset=Nk − Nq)), itself pinned against the
last rows of the square result and against chunk-by-chunk evaluation (tests/oracle_pins.py).
Tolerances as for the forward: O max-abs ≤ 1e-2, LSE max-abs ≤ 1e-3; where a few keys dominate a row
the O bound is 1e-2 plus half a bf16 ulp of the exact value (bf16 storage of |O| up to 4).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 1e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import io_aware_exact_18_amd as fa
    fa.library()
    yield


def fa():
    import io_aware_exact_18_amd as m
    return m


def _half_ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -134)


def _check(q, k, v, o, lse, causal, scale, o_tol=None):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o, lse = o.cpu(), lse.cpu()
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = oracle.attention_head_fwd64(
                q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy(),
                causal, scale, q_offset=Nk - Nq)
            og = o[b, h].double().numpy()
            lg = lse[b, h].double().numpy()
            assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
            err = np.abs(og - o_ref)
            if o_tol == "bf16_store":
                assert np.all(err <= O_TOL + _half_ulp_bf16(o_ref)), (b, h, float(err.max()))
            else:
                assert err.max() <= O_TOL, (b, h, float(err.max()))
            assert np.abs(lg - l_ref).max() <= LSE_TOL, (b, h, float(np.abs(lg - l_ref).max()))
            worst_o = max(worst_o, float(err.max()))
            worst_l = max(worst_l, float(np.abs(lg - l_ref).max()))
    return worst_o, worst_l


def _run(q, k, v, causal, scale, workspace=None):
    dev = "cuda"
    o, lse = fa().decode(q.to(dev), k.to(dev), v.to(dev), causal, scale, workspace)
    torch.cuda.synchronize()
    return o, lse


# Shapes: single key, ragged tiles (Nk not a multiple of 32), Nq up to 32, caches long enough to be
# split into several chunks (≥ 512 keys with B·H = 2) with a ragged last chunk, every head dim.
SMALL = [
    (1, 1, 64, True), (1, 5, 128, False), (1, 33, 128, True), (3, 31, 64, True),
    (8, 64, 128, True), (8, 257, 128, True), (32, 32, 128, True), (32, 300, 64, False),
    (5, 1000, 128, True), (16, 3000, 128, True), (1, 4097, 64, False), (2, 777, 64, True),
    (1, 1, 256, True), (7, 301, 256, True), (32, 1500, 256, False), (4, 2049, 256, True),
    (1, 1, 96, True), (3, 333, 96, False), (32, 1024, 96, True), (8, 2500, 96, True),
]


@pytest.mark.parametrize("Nq,Nk,d,causal", SMALL)
def test_decode_small(Nq, Nk, d, causal):
    g = torch.Generator().manual_seed(Nq * 131 + Nk + d + int(causal))
    q = torch.randn(1, 2, Nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, Nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, Nk, d, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, causal, scale)
    _check(q, k, v, o, lse, causal, scale)


@pytest.mark.parametrize("step_log2", [16.0, 6.0, -6.0])
def test_decode_rising_row_maximum(step_log2):
    """Scores that rise (or fall) by step_log2 (base 2) per 256 keys: the reference maximum moves
    inside chunks and the chunk merge weights differ by large factors."""
    B, H, Nq, Nk, d = 1, 2, 4, 2600, 128
    g = torch.Generator().manual_seed(int(step_log2) + 100)
    scale = 1.0 / math.sqrt(d)
    q = torch.randn(B, H, Nq, d, generator=g)
    k = torch.randn(B, H, Nk, d, generator=g)
    v = torch.randn(B, H, Nk, d, generator=g)
    q[..., 0] = 64.0
    t = (torch.arange(Nk) // 256).to(torch.float32)
    k[..., 0] = (step_log2 * math.log(2.0) / (scale * 64.0)) * t.view(1, 1, Nk)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = _run(q, k, v, True, scale)
    _check(q, k, v, o, lse, True, scale, o_tol="bf16_store")


def test_decode_deterministic_and_workspace_reuse():
    """Two calls give bitwise-equal results; a caller-provided workspace serves a larger call and then
    a smaller one without being cleared (its contents need no initialisation)."""
    g = torch.Generator().manual_seed(7)
    d = 128
    q = torch.randn(2, 3, 8, d, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, 3, 2000, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(2, 3, 2000, d, generator=g).to(torch.bfloat16).cuda()
    ws = torch.full((fa().decode_workspace_bytes(2, 3, 8, 2000, d),), 0x7F, dtype=torch.uint8,
                    device="cuda")  # NaN-like garbage in every fp32 slot
    o1, l1 = fa().decode(q, k, v, True, workspace=ws)
    o2, l2 = fa().decode(q, k, v, True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = fa().decode(q[:, :, :2].contiguous(), k[:, :, :900].contiguous(),
                         v[:, :, :900].contiguous(), False, workspace=ws)
    o4, l4 = fa().decode(q[:, :, :2].contiguous(), k[:, :, :900].contiguous(),
                         v[:, :, :900].contiguous(), False)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    _check(q[:, :, :2].cpu(), k[:, :, :900].cpu(), v[:, :, :900].cpu(), o3, l3, False,
           1.0 / math.sqrt(d))


def test_decode_rejects_bad_arguments():
    q = torch.zeros(1, 1, 33, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa().FaError):
        fa().decode(q, k, k, True)  # Nq > 32
    q = torch.zeros(1, 1, 9, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa().FaError):
        fa().decode(q, k, k, True)  # Nk < Nq


@pytest.mark.parametrize("name", ["decode_32k", "specdec_32k"])
def test_decode_workload_full(name):
    """The decoding workloads at full size, every head against the oracle."""
    w = workloads.DECODE_WORKLOADS[name]
    inp = workloads.make_decode_inputs(name)
    o, lse = _run(inp["q"], inp["k"], inp["v"], w.causal, w.scale)
    worst = _check(inp["q"], inp["k"], inp["v"], o, lse, w.causal, w.scale)
    print(f"{name}: worst |O - O*| = {worst[0]:.3g}, |LSE - LSE*| = {worst[1]:.3g}")


@pytest.mark.parametrize("scale", [0.03, 0.4])
def test_decode_other_softmax_scales(scale):
    """Flatter and sharper rows than 1/√d: the scale enters the split kernel's exponentials."""
    g = torch.Generator().manual_seed(int(scale * 1000))
    q = torch.randn(1, 2, 5, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, 1500, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, 1500, 128, generator=g).to(torch.bfloat16)
    o, lse = _run(q, k, v, True, scale)
    _check(q, k, v, o, lse, True, scale, o_tol="bf16_store")


def test_decode_largest_head():
    """The largest cache one head may hold at d = 128: the kernels address a head with 32-bit byte
    offsets and the library accepts (Nk + 256) · d · 2 < 2^31, so Nk = 2^23 − 257 keys (2 GiB each for
    K and V, a ragged last tile and chunk).  Four queries, causal, checked against the oracle."""
    Nq, Nk, d = 4, (1 << 23) - 257, 128
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device="cuda").manual_seed(23)
    q = torch.randn(1, 1, Nq, d, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(1, 1, Nk, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(1, 1, Nk, d, device="cuda", generator=g).to(torch.bfloat16)
    o, lse = fa().decode(q, k, v, True, scale)
    torch.cuda.synchronize()
    worst = _check(q.cpu(), k.cpu(), v.cpu(), o, lse, True, scale)
    print(f"Nk = {Nk}: worst |O - O*| = {worst[0]:.3g}, |LSE - LSE*| = {worst[1]:.3g}")
