"""Seeded random shapes through every compute entry point, against the fp64 CPU oracle.

Each case draws B, H, N, d, the causal flag and the softmax scale (0.03 to 0.15, around the 1/√d of
these head dimensions) from a fixed seed, with N up to 3000 so the oracle finishes in seconds.  It
checks the bf16 forward and backward, the split forward and backward (which run their split kernels
on the shapes that have too few query tiles), and the FP8 forward, at the same bounds as the
fixed-shape tests: O max-abs ≤ 1e-2, LSE max-abs ≤ 1e-3, gradients' relative Frobenius error ≤ 2e-2;
FP8: O max-abs ≤ 6e-2.
"""

import math
import random

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL, GRAD_TOL, FP8_O_TOL = 1e-2, 1e-3, 2e-2, 6e-2


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


def _rel_fro(got, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (den if den > 0 else 1.0)


def _case(i):
    rnd = random.Random(7000 + i)
    B, H = rnd.randint(1, 2), rnd.randint(1, 3)
    N = rnd.choice([rnd.randint(1, 200), rnd.randint(200, 1200), rnd.randint(1025, 3000)])
    d = rnd.choice([64, 96, 128, 256])
    causal = rnd.random() < 0.6
    scale = math.exp(rnd.uniform(math.log(0.03), math.log(0.15)))
    return B, H, N, d, causal, scale


CASES = [_case(i) for i in range(64)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_shape_all_paths(case):
    B, H, N, d, causal, scale = CASES[case]
    g = torch.Generator().manual_seed(9000 + case)
    q, k, v, do = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16) for _ in range(4))
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = fa().fwd(qd, kd, vd, causal, scale)
    dq, dk, dv = fa().bwd(qd, kd, vd, o, lse, dod, causal, scale)
    o_s, l_s = fa().fwd_split(qd, kd, vd, causal, scale)
    g_s = fa().bwd_split(qd, kd, vd, o, lse, dod, causal, scale)
    torch.cuda.synchronize()
    split = fa().fwd_split_workspace_bytes(B, H, N, d, causal) > 0
    worst = {"O": 0.0, "LSE": 0.0, "grad": 0.0}
    for h in range(B * H):
        b, hh = divmod(h, H)
        q64, k64, v64, do64 = (_np64(x[b, hh]) for x in (q, k, v, do))
        o_ref, l_ref = oracle.attention_head_fwd64(q64, k64, v64, causal, scale)
        refs = oracle.attention_head_bwd64(q64, k64, v64, do64, causal, scale)
        for oo, ll in ((o, lse), (o_s, l_s)):
            e_o = float(np.abs(_np64(oo[b, hh]) - o_ref).max())
            e_l = float(np.abs(_np64(ll[b, hh]) - l_ref).max())
            assert e_o <= O_TOL and e_l <= LSE_TOL, (CASES[case], h, e_o, e_l)
            worst["O"], worst["LSE"] = max(worst["O"], e_o), max(worst["LSE"], e_l)
        for grads in ((dq, dk, dv), g_s):
            for got, ref, name in zip(grads, refs, ("dq", "dk", "dv")):
                e = _rel_fro(_np64(got[b, hh]), ref)
                assert e <= GRAD_TOL, (CASES[case], h, name, e)
                worst["grad"] = max(worst["grad"], e)
    # the FP8 forward on the same shape, with e4m3 inputs quantised from the same draws
    inp = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        inp[name + "8"], inp["s" + name] = workloads.quantize_e4m3(x.float())
    o8, l8 = fa().fwd_fp8(*(inp[n + "8"].cuda() for n in "qkv"), inp["sq"], inp["sk"], inp["sv"],
                          causal, scale)
    torch.cuda.synchronize()
    deq = [workloads.dequantized64(inp[n + "8"], inp["s" + n]) for n in "qkv"]
    for h in range(B * H):
        b, hh = divmod(h, H)
        o_ref, _ = oracle.attention_head_fwd64(*(x[b, hh].numpy() for x in deq), causal, scale)
        e8 = float(np.abs(_np64(o8[b, hh]) - o_ref).max())
        assert e8 <= FP8_O_TOL, (CASES[case], h, e8)
    print(f"PARITY random {CASES[case]} split={split}: O {worst['O']:.3g} LSE {worst['LSE']:.3g} "
          f"grad {worst['grad']:.3g}")
