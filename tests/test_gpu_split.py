"""GPU parity of the key-range split forward, backward and FP8 forward (fa_fwd_split, fa_bwd_split,
fa_fwd_fp8_split) against the fp64 CPU oracle, and against the unsplit calls.

The split only changes how a query tile's keys are grouped: each segment's partial result is merged
by its softmax mass, so the bounds are those of the forward (O max-abs ≤ 1e-2, LSE max-abs ≤ 1e-3),
and the split and unsplit outputs of one input differ only by rounding order.
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
    fa.library()  # fail loudly if libfa.so is missing
    yield


def fa():
    import io_aware_exact_18_amd as m
    return m


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _inputs(B, H, N, d, seed, device="cpu"):
    g = torch.Generator(device=device).manual_seed(seed)
    return [torch.randn(B, H, N, d, generator=g, device=device).to(torch.bfloat16) for _ in range(3)]


def _check_rows(q, k, v, o, lse, causal, scale, rows=None):
    """Every head (all rows, or the given row blocks) against the oracle; returns the worst errors."""
    B, H, N, d = q.shape
    worst_o = worst_l = 0.0
    for h in range(B * H):
        b, hh = divmod(h, H)
        q64, k64, v64 = (_np64(x[b, hh]) for x in (q, k, v))
        o_c, l_c = o[b, hh].cpu(), lse[b, hh].cpu()
        for r0, r1 in (rows or [(0, N)]):
            kend = r1 if causal else N
            o_ref, l_ref = oracle.attention_head_fwd64(q64[r0:r1], k64[:kend], v64[:kend], causal,
                                                      scale, q_offset=r0)
            err_o = float(np.abs(_np64(o_c[r0:r1]) - o_ref).max())
            err_l = float(np.abs(_np64(l_c[r0:r1]) - l_ref).max())
            assert err_o <= O_TOL, (h, r0, err_o)
            assert err_l <= LSE_TOL, (h, r0, err_l)
            worst_o, worst_l = max(worst_o, err_o), max(worst_l, err_l)
    return worst_o, worst_l


SPLIT_SMALL = [(1, 1, n, d, c) for d in (64, 96, 128) for c in (False, True)
               for n in (1025, 1100, 2000, 3001, 4096)]


@pytest.mark.parametrize("B,H,N,d,causal", SPLIT_SMALL)
def test_fwd_split_small(B, H, N, d, causal):
    """One head long enough to be split (more than 16 key tiles), ragged lengths included: N = 1025
    leaves a last segment holding one key."""
    assert fa().fwd_split_workspace_bytes(B, H, N, d, causal) > 0  # the split path runs
    q, k, v = _inputs(B, H, N, d, seed=N * 3 + d + int(causal))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa().fwd_split(q.cuda(), k.cuda(), v.cuda(), causal, scale)
    torch.cuda.synchronize()
    worst = _check_rows(q, k, v, o, lse, causal, scale)
    print(f"PARITY fwd_split {B}x{H}x{N}x{d} causal={causal}: O {worst[0]:.3g} LSE {worst[1]:.3g}")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_split_several_heads(causal):
    """Three heads of 5000 keys (120 query tiles in all, so split): every head against the oracle."""
    B, H, N, d = 1, 3, 5000, 128
    assert fa().fwd_split_workspace_bytes(B, H, N, d, causal) > 0
    q, k, v = _inputs(B, H, N, d, seed=5000 + int(causal))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa().fwd_split(q.cuda(), k.cuda(), v.cuda(), causal, scale)
    torch.cuda.synchronize()
    worst = _check_rows(q, k, v, o, lse, causal, scale)
    print(f"PARITY fwd_split {B}x{H}x{N}x{d} causal={causal}: O {worst[0]:.3g} LSE {worst[1]:.3g}")


@pytest.mark.parametrize("N,d", [(16384, 128), (65536, 64)])
def test_fwd_split_long_head_matches_unsplit(N, d):
    """A single long causal head: the split and unsplit forwards agree within the O bound (each segment
    rounds its probabilities to bf16 against its own reference maximum, so the rounded weights, and
    O, differ at that level) and LSE within 2e-5 (fp32 sums); row blocks at the start, the middle and
    the end of the split result match the oracle; repeated calls are bit-identical."""
    B, H, causal = 1, 1, True
    assert fa().fwd_split_workspace_bytes(B, H, N, d, causal) > 0
    q, k, v = _inputs(B, H, N, d, seed=N + d, device="cuda")
    scale = 1.0 / math.sqrt(d)
    o_s, l_s = fa().fwd_split(q, k, v, causal, scale)
    o_u, l_u = fa().fwd(q, k, v, causal, scale)
    o_s2, l_s2 = fa().fwd_split(q, k, v, causal, scale)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_s2) and torch.equal(l_s, l_s2)  # deterministic
    diff_o = (o_s.float() - o_u.float()).abs()
    assert float(diff_o.max()) <= O_TOL
    assert float((l_s - l_u).abs().max()) <= 2e-5
    rows = [(0, 8), (N // 2 - 5, N // 2 + 3), (N - 8, N)]
    worst = _check_rows(q.cpu(), k.cpu(), v.cpu(), o_s, l_s, causal, scale, rows=rows)
    print(f"PARITY fwd_split 1x1x{N}x{d} causal: O {worst[0]:.3g} LSE {worst[1]:.3g}; "
          f"vs unsplit O {float(diff_o.max()):.3g}")


def test_fwd_split_unsplit_shapes_equal_fwd():
    """Shapes that are not split need no workspace, and fa_fwd_split then gives fa_fwd's output bit for
    bit: enough query tiles (2048), at most 16 key tiles (N ≤ 1024), head dimension 256."""
    for B, H, N, d, causal in ((16, 16, 1024, 64, True), (2, 4, 1000, 128, False),
                               (1, 1, 1024, 96, True), (1, 1, 3000, 256, True)):
        assert fa().fwd_split_workspace_bytes(B, H, N, d, causal) == 0, (B, H, N, d)
        q, k, v = _inputs(B, H, N, d, seed=B * H + N, device="cuda")
        o_u, l_u = fa().fwd(q, k, v, causal)
        o_s, l_s = fa().fwd_split(q, k, v, causal,
                                  workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_u) and torch.equal(l_s, l_u), (B, H, N, d)


def test_fwd_split_workspace_reuse_with_smaller_shape():
    """One workspace, two calls in a row, the second on a smaller split shape: the stale partial results
    of the first call are never read."""
    q1, k1, v1 = _inputs(1, 1, 6000, 128, seed=61, device="cuda")
    q2, k2, v2 = _inputs(1, 1, 2100, 128, seed=62, device="cuda")
    need1 = fa().fwd_split_workspace_bytes(1, 1, 6000, 128, True)
    need2 = fa().fwd_split_workspace_bytes(1, 1, 2100, 128, True)
    assert need1 >= need2 > 0
    ws = torch.empty(need1, dtype=torch.uint8, device="cuda")
    fa().fwd_split(q1, k1, v1, True, workspace=ws)
    o2, l2 = fa().fwd_split(q2, k2, v2, True, workspace=ws)
    torch.cuda.synchronize()
    _check_rows(q2.cpu(), k2.cpu(), v2.cpu(), o2, l2, True, 1.0 / math.sqrt(128))


# ------------------------------------------------------------------------------------------------
# Split backward (fa_bwd_split).  Each gradient is a sum over keys (dQ) or queries (dK, dV); the
# split only groups those sums differently, so the oracle bound is the backward's (relative Frobenius
# error ≤ 2e-2) and split and unsplit gradients agree to fp32 summation order plus one bf16 rounding.

GRAD_TOL, SAME_TOL = 2e-2, 4e-3


def _rel_fro(got, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (den if den > 0 else 1.0)


def _bwd_both(q, k, v, do, causal, scale, workspace=None):
    """Forward, then the split and the unsplit backward of the same inputs (device tensors)."""
    o, lse = fa().fwd(q, k, v, causal, scale)
    split = fa().bwd_split(q, k, v, o, lse, do, causal, scale, workspace=workspace)
    plain = fa().bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    return split, plain


def _check_bwd_oracle(q, k, v, do, grads, causal, scale):
    B, H, N, d = q.shape
    worst = 0.0
    for h in range(B * H):
        b, hh = divmod(h, H)
        ref = oracle.attention_head_bwd64(*(_np64(x[b, hh]) for x in (q, k, v, do)), causal, scale)
        for got, r, name in zip(grads, ref, ("dq", "dk", "dv")):
            g = _np64(got[b, hh])
            assert np.all(np.isfinite(g)), (h, name)
            e = _rel_fro(g, r)
            assert e <= GRAD_TOL, (h, name, e)
            worst = max(worst, e)
    return worst


def _check_same(split, plain):
    worst = 0.0
    for s, p, name in zip(split, plain, ("dq", "dk", "dv")):
        e = _rel_fro(_np64(s), _np64(p))
        assert e <= SAME_TOL, (name, e)
        worst = max(worst, e)
    return worst


SPLIT_BWD = [(1, 1, n, d, c) for d in (64, 96, 128) for c in (False, True) for n in (1025, 2000, 3001)]


@pytest.mark.parametrize("B,H,N,d,causal", SPLIT_BWD)
def test_bwd_split_small(B, H, N, d, causal):
    """One head long enough to be split, ragged lengths included: dQ, dK, dV against the oracle and
    against the unsplit backward."""
    assert fa().bwd_split_workspace_bytes(B, H, N, d, causal) > fa().bwd_workspace_bytes(B, H, N, d)
    q, k, v = _inputs(B, H, N, d, seed=7 * N + d + int(causal))
    do = _inputs(B, H, N, d, seed=7 * N + d + 99)[0]
    scale = 1.0 / math.sqrt(d)
    split, plain = _bwd_both(q.cuda(), k.cuda(), v.cuda(), do.cuda(), causal, scale)
    e_o = _check_bwd_oracle(q, k, v, do, split, causal, scale)
    e_s = _check_same(split, plain)
    print(f"PARITY bwd_split {B}x{H}x{N}x{d} causal={causal}: oracle {e_o:.3g} vs unsplit {e_s:.3g}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_split_several_heads(causal):
    B, H, N, d = 1, 3, 5000, 128
    assert fa().bwd_split_workspace_bytes(B, H, N, d, causal) > fa().bwd_workspace_bytes(B, H, N, d)
    q, k, v = _inputs(B, H, N, d, seed=5100 + int(causal))
    do = _inputs(B, H, N, d, seed=5200)[0]
    scale = 1.0 / math.sqrt(d)
    split, plain = _bwd_both(q.cuda(), k.cuda(), v.cuda(), do.cuda(), causal, scale)
    e_o = _check_bwd_oracle(q, k, v, do, split, causal, scale)
    e_s = _check_same(split, plain)
    print(f"PARITY bwd_split {B}x{H}x{N}x{d} causal={causal}: oracle {e_o:.3g} vs unsplit {e_s:.3g}")


def test_bwd_split_long_head():
    """One causal head of 16384 keys: split against unsplit gradients, dQ row blocks at the start, the
    middle and the end against the oracle's row-restricted form, the exact sums Σ dV = Σ dO and
    Σ dK = 0, and bit-identical repeated calls."""
    B, H, N, d, causal = 1, 1, 16384, 128, True
    q, k, v = _inputs(B, H, N, d, seed=16384, device="cuda")
    do = _inputs(B, H, N, d, seed=16385, device="cuda")[0]
    scale = 1.0 / math.sqrt(d)
    split, plain = _bwd_both(q, k, v, do, causal, scale)
    o, lse = fa().fwd(q, k, v, causal, scale)
    again = fa().bwd_split(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(split, again))
    e_s = _check_same(split, plain)
    q64, k64, v64, do64 = (_np64(x[0, 0]) for x in (q, k, v, do))
    dq_c = split[0][0, 0].cpu()
    for r0 in (0, N // 2 - 4, N - 8):
        rows = list(range(r0, r0 + 8))
        ref = oracle.attention_rows_dq64(q64, k64, v64, do64, rows, causal, scale)
        assert _rel_fro(_np64(dq_c[r0:r0 + 8]), ref) <= GRAD_TOL, r0
    dq, dk, dv = split
    sdv, sdo = dv.double().sum(dim=2), do.double().sum(dim=2)
    assert ((sdv - sdo).norm(dim=-1) / sdo.norm(dim=-1)).max().item() <= GRAD_TOL
    assert (dk.double().sum(dim=2).norm(dim=-1) / dk.double().norm(dim=(2, 3))).max().item() <= GRAD_TOL
    print(f"PARITY bwd_split 1x1x{N}x{d} causal: vs unsplit {e_s:.3g}")


def test_bwd_split_unsplit_shapes_equal_bwd():
    """Shapes that are not split need fa_bwd's workspace only, and fa_bwd_split then gives fa_bwd's
    gradients bit for bit."""
    for B, H, N, d, causal in ((16, 16, 1024, 64, True), (1, 1, 1024, 96, False),
                               (1, 1, 3000, 256, True)):
        assert fa().bwd_split_workspace_bytes(B, H, N, d, causal) == fa().bwd_workspace_bytes(B, H, N, d)
        q, k, v = _inputs(B, H, N, d, seed=B * H + N + 1, device="cuda")
        do = _inputs(B, H, N, d, seed=B * H + N + 2, device="cuda")[0]
        split, plain = _bwd_both(q, k, v, do, causal, 1.0 / math.sqrt(d))
        assert all(torch.equal(a, b) for a, b in zip(split, plain)), (B, H, N, d)


def test_bwd_split_workspace_reuse_with_smaller_shape():
    """One workspace, two calls in a row, the second on a smaller split shape."""
    need = fa().bwd_split_workspace_bytes(1, 1, 6000, 128, True)
    assert need >= fa().bwd_split_workspace_bytes(1, 1, 2100, 64, True) > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    q, k, v = _inputs(1, 1, 6000, 128, seed=71, device="cuda")
    do = _inputs(1, 1, 6000, 128, seed=72, device="cuda")[0]
    _bwd_both(q, k, v, do, True, 1.0 / math.sqrt(128), workspace=ws)
    q, k, v = _inputs(1, 1, 2100, 64, seed=73)
    do = _inputs(1, 1, 2100, 64, seed=74)[0]
    split, plain = _bwd_both(q.cuda(), k.cuda(), v.cuda(), do.cuda(), True, 0.125, workspace=ws)
    _check_bwd_oracle(q, k, v, do, split, True, 0.125)
    _check_same(split, plain)


# ------------------------------------------------------------------------------------------------
# Split FP8 forward (fa_fwd_fp8_split): the FP8 forward's bounds against the oracle on the values the
# e4m3 codes stand for (O max-abs ≤ 6e-2, LSE max-abs ≤ 5e-2, as in the fixed-shape FP8 tests).

FP8_O_TOL, FP8_LSE_TOL = 6e-2, 5e-2


def _fp8_inputs(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    out = {}
    for name in ("q", "k", "v"):
        out[name + "8"], out["s" + name] = workloads.quantize_e4m3(torch.randn(B, H, N, d, generator=g))
    return out


def _check_fp8_rows(inp, o, lse, causal, scale, rows=None):
    q, k, v = (workloads.dequantized64(inp[n + "8"], inp["s" + n]) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    worst_o = worst_l = 0.0
    for h in range(B * H):
        b, hh = divmod(h, H)
        o_c, l_c = o[b, hh].cpu(), lse[b, hh].cpu()
        for r0, r1 in (rows or [(0, N)]):
            kend = r1 if causal else N
            o_ref, l_ref = oracle.attention_head_fwd64(q[b, hh, r0:r1].numpy(), k[b, hh, :kend].numpy(),
                                                      v[b, hh, :kend].numpy(), causal, scale,
                                                      q_offset=r0)
            e_o = float(np.abs(_np64(o_c[r0:r1]) - o_ref).max())
            e_l = float(np.abs(_np64(l_c[r0:r1]) - l_ref).max())
            assert e_o <= FP8_O_TOL and e_l <= FP8_LSE_TOL, (h, r0, e_o, e_l)
            worst_o, worst_l = max(worst_o, e_o), max(worst_l, e_l)
    return worst_o, worst_l


def _run_fp8(fn, inp, causal, scale):
    o, lse = fn(*(inp[n + "8"].cuda() for n in ("q", "k", "v")), inp["sq"], inp["sk"], inp["sv"],
                causal, scale)
    torch.cuda.synchronize()
    return o, lse


SPLIT_FP8 = [(1, 1, n, d, c) for d in (64, 96, 128) for c in (False, True) for n in (1025, 3001)]


@pytest.mark.parametrize("B,H,N,d,causal", SPLIT_FP8)
def test_fwd_fp8_split_small(B, H, N, d, causal):
    assert fa().fwd_split_workspace_bytes(B, H, N, d, causal) > 0
    inp = _fp8_inputs(B, H, N, d, seed=11 * N + d + int(causal))
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fp8(fa().fwd_fp8_split, inp, causal, scale)
    worst = _check_fp8_rows(inp, o, lse, causal, scale)
    o_u, l_u = _run_fp8(fa().fwd_fp8, inp, causal, scale)
    d_o = float((o.float() - o_u.float()).abs().max())
    assert d_o <= FP8_O_TOL
    print(f"PARITY fwd_fp8_split {B}x{H}x{N}x{d} causal={causal}: O {worst[0]:.3g} "
          f"LSE {worst[1]:.3g}; vs unsplit O {d_o:.3g}")


def test_fwd_fp8_split_long_head():
    """One causal head of 16384 keys: split against unsplit FP8 outputs (within the FP8 bounds), row
    blocks against the oracle, bit-identical repeated calls."""
    B, H, N, d, causal = 1, 1, 16384, 128, True
    inp = _fp8_inputs(B, H, N, d, seed=16384 * 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fp8(fa().fwd_fp8_split, inp, causal, scale)
    o2, l2 = _run_fp8(fa().fwd_fp8_split, inp, causal, scale)
    assert torch.equal(o, o2) and torch.equal(l2, lse)
    o_u, l_u = _run_fp8(fa().fwd_fp8, inp, causal, scale)
    assert float((o.float() - o_u.float()).abs().max()) <= FP8_O_TOL
    # each segment rounds P to e4m3 against its own reference maximum, so the sums differ at the
    # level of that rounding; both are held to the oracle bound below
    assert float((lse - l_u).abs().max()) <= FP8_LSE_TOL
    worst = _check_fp8_rows(inp, o, lse, causal, scale,
                            rows=[(0, 8), (N // 2 - 4, N // 2 + 4), (N - 8, N)])
    print(f"PARITY fwd_fp8_split 1x1x{N}x{d} causal: O {worst[0]:.3g} LSE {worst[1]:.3g}")


def test_fwd_fp8_split_unsplit_shapes_equal_fwd_fp8():
    for B, H, N, d in ((4, 8, 2048, 128), (1, 1, 1024, 64), (1, 1, 3000, 256)):
        assert fa().fwd_split_workspace_bytes(B, H, N, d, True) == 0
        inp = _fp8_inputs(B, H, N, d, seed=B * H + N)
        a = _run_fp8(fa().fwd_fp8, inp, True, 1.0 / math.sqrt(d))
        b = _run_fp8(fa().fwd_fp8_split, inp, True, 1.0 / math.sqrt(d))
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (B, H, N, d)
