"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the bench and the smoke check: it feeds the same input values to the
CPU oracle and to the HIP path.  It holds no attention arithmetic — only shapes, seeded random draws and
the storage formats the inputs are handed over in (bf16 round-to-nearest-even; OCP e4m3fn with a
per-tensor fp32 scale).

Workloads (shapes [B, H, N, d], d innermost; scale 1/√d):

========  =====================  ======  ========================================================
name      B, H, N, d             causal  what runs
========  =====================  ======  ========================================================
fwd_small 1, 2, 256, 64          no      forward only, bf16
d64_2k    8, 16, 2048, 64        no      forward + backward, bf16
causal_4k 4, 32, 4096, 128       yes     forward + backward, bf16 (the throughput workload)
long_16k  1, 32, 16384, 128      yes     forward + backward, bf16, one ×8 key per 1024-key block
fp8_8k    4, 32, 8192, 128       yes     forward only, e4m3 Q/K/V with per-tensor scales, O bf16
d256_4k   4, 16, 4096, 256       yes     forward + backward, bf16, head dimension 256 (the FLOPs of
                                         causal_4k with half the heads, each twice as wide)
d96_4k    4, 32, 4096, 96        yes     forward + backward, bf16, head dimension 96
fp8bwd_8k 4, 32, 8192, 128       yes     fp8 forward + backward: e4m3 Q/K/V as fp8_8k, dO bf16
fp8_d64_8k 4, 32, 8192, 64       yes     fp8 forward only, as fp8_8k at head dimension 64
fp8_d96_8k 4, 32, 8192, 96       yes     fp8 forward only, as fp8_8k at head dimension 96
fp8_d256_8k 4, 16, 8192, 256     yes     fp8 forward only, head dimension 256 (the FLOPs of fp8_8k)
onehead_32k 1, 1, 32768, 128     yes     forward + backward, bf16, one head: too few query tiles to
                                         fill the device unsplit (the split forward and backward)
========  =====================  ======  ========================================================

Decoding workloads (queries [B, H, Nq, d] against a key/value cache [B, H, Nk, d]; the queries are the
last Nq positions of the sequence, so with the causal mask query i may use keys j ≤ Nk − Nq + i):

===========  ==========================  ======  ===================================================
name         B, H, Nq, Nk, d             causal  what runs
===========  ==========================  ======  ===================================================
decode_32k   4, 32, 1, 32768, 128        yes     one new token per sequence, bf16
specdec_32k  4, 32, 8, 32768, 128        yes     8 draft tokens verified at once (speculative), bf16
===========  ==========================  ======  ===================================================

Seeds: tensor t of workload c uses ``torch.Generator().manual_seed(1000*c + t)`` with c the workload
number 1..14 and t = 0 (Q), 1 (K), 2 (V), 3 (dO), 4 (positions of the enlarged keys).  Values are drawn
as float32 N(0, 1) on the CPU and rounded to the storage type, so every consumer sees identical inputs.
"""

import math
from dataclasses import dataclass

import torch

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    backward: bool
    fp8: bool = False
    large_keys: bool = False

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    def shape(self, B=None, H=None, N=None):
        return (self.B if B is None else B, self.H if H is None else H,
                self.N if N is None else N, self.d)

    def fwd_flops(self, B=None, H=None, N=None):
        """Forward FLOPs by the usual convention: 4·B·H·N²·d, halved when causal."""
        b, h, n, d = self.shape(B, H, N)
        f = 4.0 * b * h * n * n * d
        return f / 2 if self.causal else f

    def bwd_flops(self, B=None, H=None, N=None):
        """Backward FLOPs by the usual convention: 2.5 × the forward."""
        return 2.5 * self.fwd_flops(B, H, N)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(1, "fwd_small", 1, 2, 256, 64, causal=False, backward=False),
        Workload(2, "d64_2k", 8, 16, 2048, 64, causal=False, backward=True),
        Workload(3, "causal_4k", 4, 32, 4096, 128, causal=True, backward=True),
        Workload(4, "long_16k", 1, 32, 16384, 128, causal=True, backward=True, large_keys=True),
        Workload(5, "fp8_8k", 4, 32, 8192, 128, causal=True, backward=False, fp8=True),
        Workload(8, "d256_4k", 4, 16, 4096, 256, causal=True, backward=True),
        Workload(9, "d96_4k", 4, 32, 4096, 96, causal=True, backward=True),
        Workload(10, "fp8bwd_8k", 4, 32, 8192, 128, causal=True, backward=True, fp8=True),
        Workload(11, "fp8_d64_8k", 4, 32, 8192, 64, causal=True, backward=False, fp8=True),
        Workload(12, "fp8_d96_8k", 4, 32, 8192, 96, causal=True, backward=False, fp8=True),
        Workload(13, "fp8_d256_8k", 4, 16, 8192, 256, causal=True, backward=False, fp8=True),
        Workload(14, "onehead_32k", 1, 1, 32768, 128, causal=True, backward=True),
    ]
}


@dataclass(frozen=True)
class DecodeWorkload:
    number: int
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    def q_shape(self, B=None, H=None):
        return (self.B if B is None else B, self.H if H is None else H, self.Nq, self.d)

    def kv_shape(self, B=None, H=None, Nk=None):
        return (self.B if B is None else B, self.H if H is None else H,
                self.Nk if Nk is None else Nk, self.d)

    def kv_bytes(self, B=None, H=None, Nk=None):
        """Bytes of the bf16 key and value cache: what one decode step must read at least once."""
        b, h, n, d = self.kv_shape(B, H, Nk)
        return 2 * b * h * n * d * 2


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload(6, "decode_32k", 4, 32, 1, 32768, 128, causal=True),
        DecodeWorkload(7, "specdec_32k", 4, 32, 8, 32768, 128, causal=True),
    ]
}


def make_decode_inputs(name, B=None, H=None, Nk=None):
    """Inputs of a decoding workload as CPU bf16 tensors {"q", "k", "v"}, optionally at a reduced B,
    H or cache length Nk (same seeds)."""
    w = DECODE_WORKLOADS[name]
    c = w.number
    return {
        "q": to_bf16(randn_f32(w.q_shape(B, H), 1000 * c + 0)),
        "k": to_bf16(randn_f32(w.kv_shape(B, H, Nk), 1000 * c + 1)),
        "v": to_bf16(randn_f32(w.kv_shape(B, H, Nk), 1000 * c + 2)),
    }


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def randn_f32(shape, seed):
    """float32 N(0,1) draws from a CPU generator seeded with ``seed``."""
    return torch.randn(shape, generator=_gen(seed), dtype=torch.float32)


def to_bf16(x):
    """Round float32 to bfloat16, round-to-nearest-even (torch's cast)."""
    return x.to(torch.bfloat16)


def enlarge_keys(k, seed, block=1024, factor=8.0):
    """Multiply one key row per ``block`` consecutive keys by ``factor`` (a power of two: exact).

    For each (b, h) and each key block t, the row block·t + u is chosen with u uniform over the block
    (the last block may be shorter), drawn from a generator seeded with ``seed``.
    """
    b_, h_, n, _ = k.shape
    g = _gen(seed)
    out = k.clone()
    n_blocks = (n + block - 1) // block
    for b in range(b_):
        for h in range(h_):
            for t in range(n_blocks):
                width = min(block, n - t * block)
                u = int(torch.randint(0, width, (1,), generator=g))
                out[b, h, t * block + u, :] *= factor
    return out


def round_e4m3(x):
    """float32 → e4m3fn codes: e4m3(RNE(clamp(x, ±448))), saturating at the largest finite value.
    The clamp keeps torch's cast from turning values just past 448 into NaN."""
    return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)


def quantize_e4m3(x):
    """Per-tensor e4m3fn quantisation: s = amax|x| / 448 (fp32), x8 = e4m3(RNE(clamp(x / s, ±448))).

    Returns (x8 as torch.float8_e4m3fn, s as a Python float).
    """
    amax = float(x.abs().max())
    s = amax / E4M3_MAX if amax > 0 else 1.0
    s = float(torch.tensor(s, dtype=torch.float32))
    x8 = round_e4m3(x / s)
    return x8, s


def make_inputs(name, B=None, H=None, N=None):
    """Inputs of a workload as CPU tensors, optionally at a reduced B, H or N (same seeds).

    bf16 workloads: {"q","k","v"} bf16 and, with a backward, "do" bf16.
    fp8 workload: {"q8","k8","v8"} float8_e4m3fn, {"sq","sk","sv"} floats (dequantised value = code·s).
    """
    w = WORKLOADS[name]
    shape = w.shape(B, H, N)
    c = w.number
    q = randn_f32(shape, 1000 * c + 0)
    k = randn_f32(shape, 1000 * c + 1)
    v = randn_f32(shape, 1000 * c + 2)
    if w.large_keys:
        k = enlarge_keys(k, 1000 * c + 4)
    out = {}
    if w.fp8:
        out["q8"], out["sq"] = quantize_e4m3(q)
        out["k8"], out["sk"] = quantize_e4m3(k)
        out["v8"], out["sv"] = quantize_e4m3(v)
    else:
        out["q"], out["k"], out["v"] = to_bf16(q), to_bf16(k), to_bf16(v)
    if w.backward:
        out["do"] = to_bf16(randn_f32(shape, 1000 * c + 3))
    return out


def dequantized64(x8, s):
    """Values the e4m3 codes stand for, in float64 (code value × per-tensor scale)."""
    return x8.to(torch.float64) * s
