"""GPU parity of the FP8 backward (fa_bwd_fp8 through the C ABI) with the fp64 oracle.

The reference is the exact gradient of attention at the dequantised inputs (code · descale), computed
by oracle.attention_head_bwd64 on the same values.  Two comparisons:
  * the backward on its own: fed the oracle's O (rounded to bf16) and LSE, dQ/dK/dV must meet the
    bf16 bound, relative Frobenius error ≤ 2e-2;
  * end to end: fed fa_fwd_fp8's own O and LSE.  The forward's e4m3-rounded probabilities make its
    LSE and O inexact (its O bound is 6e-2 max-abs); an LSE error ε scales every recomputed
    probability by e^(−ε) and an O error shifts D = dO · O, so the gradients inherit these errors.
    The bound FP8_E2E_TOL = 6e-2 is the forward's O bound carried over as a relative gradient
    error; the measured worst case is printed.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

BWD_TOL = 2e-2
FP8_E2E_TOL = 6e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import io_aware_exact_18_amd as fa
    fa.library()
    yield


def fa():
    import io_aware_exact_18_amd as m
    return m


def _rel_fro(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _case(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    out = {}
    for name in ("q", "k", "v"):
        out[name + "8"], out["s" + name] = workloads.quantize_e4m3(torch.randn(B, H, N, d, generator=g))
    out["do"] = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    return out


def _deq(inp):
    return [workloads.dequantized64(inp[n + "8"], inp["s" + n]) for n in ("q", "k", "v")]


def _oracle_heads(inp, causal, scale, heads):
    q, k, v = _deq(inp)
    B, H, N, d = q.shape
    res = {}
    for h in heads:
        b, hh = divmod(h, H)
        args = [x[b, hh].numpy() for x in (q, k, v)]
        o, lse = oracle.attention_head_fwd64(*args, causal, scale)
        grads = oracle.attention_head_bwd64(*args, inp["do"][b, hh].double().numpy(), causal, scale)
        res[h] = (o, lse, grads)
    return res


def _run_bwd8(inp, o, lse, causal, scale):
    dev = "cuda"
    dq, dk, dv = fa().bwd_fp8(inp["q8"].to(dev), inp["k8"].to(dev), inp["v8"].to(dev), inp["sq"],
                              inp["sk"], inp["sv"], o.to(dev), lse.to(dev), inp["do"].to(dev),
                              causal, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _check(grads, ref, heads, H, tol, label, inp=None, scale=None):
    """Relative Frobenius error of dQ, dK, dV per head.  With a single key (N = 1) the exact dQ and
    dK are 0 (P = 1 and D = dP, so dS = 0) and a relative error is meaningless: what the kernel
    returns there is O's bf16 rounding carried through D = dO · O, bounded per row by
    |dS| ≤ ‖dO‖ ‖O‖ 2^-8, so ‖dQ‖ ≤ scale ‖dS‖ ‖k‖ and ‖dK‖ ≤ scale ‖dS‖ ‖q‖."""
    worst = 0.0
    for h in heads:
        b, hh = divmod(h, H)
        N = grads[0].shape[2]
        for name, got, want in zip(("dq", "dk", "dv"), grads, ref[h][2]):
            gg = got[b, hh].double().numpy()
            assert np.all(np.isfinite(gg)), (label, h, name)
            if N == 1 and name != "dv":
                q, k, _ = (x[b, hh].numpy() for x in _deq(inp))
                ds = np.linalg.norm(inp["do"][b, hh].double().numpy()) * np.linalg.norm(ref[h][0])
                other = k if name == "dq" else q
                bound = scale * ds * 2.0 ** -8 * np.linalg.norm(other)
                assert np.linalg.norm(gg) <= bound, (label, h, name, np.linalg.norm(gg), bound)
                continue
            err = _rel_fro(gg, want)
            assert err <= tol, (label, h, name, err)
            worst = max(worst, err)
    print(f"{label}: worst relative Frobenius error {worst:.4g}")
    return worst


def _both(inp, causal, scale, heads):
    B, H, N, d = inp["q8"].shape
    ref = _oracle_heads(inp, causal, scale, heads)
    # The backward on its own: the oracle's O (bf16) and LSE for every head.
    o_ref = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    l_ref = torch.zeros(B, H, N, dtype=torch.float32)
    for h in heads:
        b, hh = divmod(h, H)
        o_ref[b, hh] = torch.from_numpy(ref[h][0]).to(torch.bfloat16)
        l_ref[b, hh] = torch.from_numpy(ref[h][1]).to(torch.float32)
    own = _run_bwd8(inp, o_ref, l_ref, causal, scale)
    _check(own, ref, heads, H, BWD_TOL, "fp8 backward, exact O and LSE", inp, scale)
    # End to end, from the FP8 forward's outputs.
    dev = "cuda"
    o8, lse8 = fa().fwd_fp8(inp["q8"].to(dev), inp["k8"].to(dev), inp["v8"].to(dev), inp["sq"],
                            inp["sk"], inp["sv"], causal, scale)
    e2e = _run_bwd8(inp, o8.cpu(), lse8.cpu(), causal, scale)
    _check(e2e, ref, heads, H, FP8_E2E_TOL, "fp8 forward + backward", inp, scale)


@pytest.mark.parametrize("N", [1, 17, 100, 129, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bwd_small(N, causal):
    inp = _case(1, 2, N, 128, seed=N * 17 + int(causal))
    _both(inp, causal, 1.0 / math.sqrt(128), range(2))


@pytest.mark.parametrize("d", [64, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_bwd_other_head_dims(d, causal):
    """The FP8 forward and backward together at d = 64, 96 and 256."""
    inp = _case(1, 2, 300, d, seed=5 * d + int(causal))
    _both(inp, causal, 1.0 / math.sqrt(d), range(2))


@pytest.mark.parametrize("d", [64, 96, 256])
def test_fp8_bwd_other_head_dims(d):
    """The widening and scale folding do not depend on the head dimension: the backward alone, fed
    the oracle's O and LSE, at every head dimension."""
    inp = _case(1, 2, 200, d, seed=d)
    scale = 1.0 / math.sqrt(d)
    ref = _oracle_heads(inp, True, scale, range(2))
    o_ref = torch.stack([torch.from_numpy(ref[h][0]) for h in range(2)]).unsqueeze(0)
    l_ref = torch.stack([torch.from_numpy(ref[h][1]) for h in range(2)]).unsqueeze(0)
    got = _run_bwd8(inp, o_ref.to(torch.bfloat16), l_ref.to(torch.float32), True, scale)
    _check(got, ref, range(2), 2, BWD_TOL, f"fp8 backward d={d}")


def _all_codes(B, H, N, d, offset):
    """e4m3fn codes cycling through all 254 finite codes (0x7F and 0xFF are NaN)."""
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    idx = (torch.arange(B * H * N * d) + offset) % finite.numel()
    return finite[idx].view(B, H, N, d).view(torch.float8_e4m3fn)


def test_fp8_bwd_every_code():
    """Q, K and V take every finite e4m3 value: a code widened wrongly shows in dK (through Q), dQ
    (through K) or dP (through V)."""
    B, H, N, d = 1, 1, 254, 128
    inp = {"q8": _all_codes(B, H, N, d, 0), "k8": _all_codes(B, H, N, d, 77),
           "v8": _all_codes(B, H, N, d, 151), "sq": 1.0 / 224, "sk": 1.0 / 224, "sv": 1.0 / 64,
           "do": torch.randn(B, H, N, d, generator=torch.Generator().manual_seed(3))
           .to(torch.bfloat16)}
    scale = 1.0 / math.sqrt(d)
    ref = _oracle_heads(inp, False, scale, [0])
    o_ref = torch.from_numpy(ref[0][0]).to(torch.bfloat16).view(B, H, N, d)
    l_ref = torch.from_numpy(ref[0][1]).to(torch.float32).view(B, H, N)
    got = _run_bwd8(inp, o_ref, l_ref, False, scale)
    _check(got, ref, [0], H, BWD_TOL, "fp8 backward, every code")


def test_fp8_bwd_deterministic_and_guarded():
    """Two calls give bitwise-equal gradients; nothing is written past the outputs or the workspace's
    documented size, and a workspace full of garbage on entry does not matter."""
    B, H, N, d = 1, 2, 190, 128
    inp = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in _case(B, H, N, d, 9).items()}
    scale = 1.0 / math.sqrt(d)
    o, lse = fa().fwd_fp8(inp["q8"], inp["k8"], inp["v8"], inp["sq"], inp["sk"], inp["sv"], True,
                          scale)
    lib = fa().library()
    n, guard = B * H * N * d, 4096
    ws_bytes = fa().bwd_fp8_workspace_bytes(B, H, N, d)
    outs = []
    for _ in range(2):
        bufs = [torch.full((n + guard,), 3.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        ws = torch.full((ws_bytes + guard,), 0x7F, dtype=torch.uint8, device="cuda")
        code = lib.fa_bwd_fp8(inp["q8"].data_ptr(), inp["k8"].data_ptr(), inp["v8"].data_ptr(),
                              inp["sq"], inp["sk"], inp["sv"], o.data_ptr(), lse.data_ptr(),
                              inp["do"].data_ptr(), bufs[0].data_ptr(), bufs[1].data_ptr(),
                              bufs[2].data_ptr(), ws.data_ptr(), ws_bytes, B, H, N, d, 1, scale,
                              torch.cuda.current_stream().cuda_stream)
        assert code == 0
        torch.cuda.synchronize()
        for b in bufs:
            assert bool((b[n:] == 3.0).all())
        assert bool((ws[ws_bytes:] == 0x7F).all())
        outs.append([b[:n].clone() for b in bufs])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_fp8_bwd_workload_reduced():
    """fp8bwd_8k at its own N and d with 2 heads, every head."""
    w = workloads.WORKLOADS["fp8bwd_8k"]
    inp = workloads.make_inputs("fp8bwd_8k", B=1, H=2)
    _both(inp, w.causal, w.scale, range(2))


def test_fp8_bwd_workload_full():
    """fp8bwd_8k at full size, as the bench runs it: sampled heads against the oracle, finite
    gradients everywhere."""
    w = workloads.WORKLOADS["fp8bwd_8k"]
    inp = workloads.make_inputs("fp8bwd_8k")
    dev = "cuda"
    o8, lse8 = fa().fwd_fp8(inp["q8"].to(dev), inp["k8"].to(dev), inp["v8"].to(dev), inp["sq"],
                            inp["sk"], inp["sv"], w.causal, w.scale)
    grads = _run_bwd8(inp, o8.cpu(), lse8.cpu(), w.causal, w.scale)
    for t in grads:
        assert bool(torch.isfinite(t).all())
    heads = [0, w.B * w.H - 1]
    ref = _oracle_heads(inp, w.causal, w.scale, heads)
    _check(grads, ref, heads, w.H, FP8_E2E_TOL, "fp8bwd_8k full, sampled heads")
