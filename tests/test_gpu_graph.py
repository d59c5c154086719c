"""The library under HIP graph capture.  Every entry point (forward, backward, decoding, the FP8
forward and backward, and the split forward, backward and FP8 forward on a shape they split) is
captured into one graph through the current stream and replayed.  The kernels are deterministic, so
each replay must reproduce the eager results bit for bit, also with eager work between replays and
after the captured input tensors are refilled in place.  One head of the replayed results is also
checked against the fp64 oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import io_aware_exact_18_amd as fa
    fa.library()  # fail loudly if libfa.so is missing
    yield


def fa():
    import io_aware_exact_18_amd as m
    return m


B, H, N, D, NQ = 1, 3, 333, 128, 6
NL = 1100  # one head of NL keys: 18 key tiles, split by fa_fwd_split / fa_bwd_split
SCALE = 1.0 / math.sqrt(D)
S8 = (0.011, 0.013, 0.009)  # descales of the e4m3 inputs (any positive values are valid)


def _fill(bufs, seed):
    """Refill the captured input tensors in place with new seeded values."""
    g = torch.Generator().manual_seed(seed)
    for t in bufs["bf16"] + bufs["long"]:
        t.copy_(torch.randn(t.shape, generator=g).to(torch.bfloat16))
    for t in bufs["e4m3"] + bufs["long8"]:  # e4m3 codes spread over most of the format's range
        t.copy_((torch.randn(t.shape, generator=g) * 100.0).clamp(-448.0, 448.0)
                .to(torch.float8_e4m3fn))


def _work(bufs, ws):
    """Every entry point once; outputs allocated by the binding on the current stream."""
    q, k, v, do = bufs["bf16"]
    q8, k8, v8 = bufs["e4m3"]
    o, lse = fa().fwd(q, k, v, True, SCALE)
    dq, dk, dv = fa().bwd(q, k, v, o, lse, do, True, SCALE, workspace=ws["bwd"])
    # decoding: the last NQ positions as new queries against all N keys
    od, ld = fa().decode(bufs["qdec"], k, v, True, SCALE, workspace=ws["dec"])
    o8, l8 = fa().fwd_fp8(q8, k8, v8, *S8, True, SCALE)
    g8 = fa().bwd_fp8(q8, k8, v8, *S8, o8, l8, do, True, SCALE, workspace=ws["bwd8"])
    ql, kl, vl, dol = bufs["long"]
    os_, ls_ = fa().fwd_split(ql, kl, vl, True, SCALE, workspace=ws["fsplit"])
    gs = fa().bwd_split(ql, kl, vl, os_, ls_, dol, True, SCALE, workspace=ws["bsplit"])
    o8s, l8s = fa().fwd_fp8_split(*bufs["long8"], *S8, True, SCALE, workspace=ws["fsplit8"])
    return [o, lse, dq, dk, dv, od, ld, o8, l8, *g8, os_, ls_, *gs, o8s, l8s]


def test_graph_capture_and_replay_match_eager():
    dev = torch.device("cuda:0")
    bufs = {"bf16": [torch.empty(B, H, N, D, dtype=torch.bfloat16, device=dev) for _ in range(4)],
            "e4m3": [torch.empty(B, H, N, D, dtype=torch.float8_e4m3fn, device=dev)
                     for _ in range(3)],
            "qdec": torch.empty(B, H, NQ, D, dtype=torch.bfloat16, device=dev),
            "long": [torch.empty(1, 1, NL, D, dtype=torch.bfloat16, device=dev) for _ in range(4)],
            "long8": [torch.empty(1, 1, NL, D, dtype=torch.float8_e4m3fn, device=dev)
                      for _ in range(3)]}
    ws = {"bwd": torch.empty(fa().bwd_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=dev),
          "dec": torch.empty(fa().decode_workspace_bytes(B, H, NQ, N, D), dtype=torch.uint8,
                             device=dev),
          "bwd8": torch.empty(fa().bwd_fp8_workspace_bytes(B, H, N, D), dtype=torch.uint8,
                              device=dev),
          "fsplit": torch.empty(fa().fwd_split_workspace_bytes(1, 1, NL, D, True), dtype=torch.uint8,
                                device=dev),
          "bsplit": torch.empty(fa().bwd_split_workspace_bytes(1, 1, NL, D, True), dtype=torch.uint8,
                                device=dev),
          "fsplit8": torch.empty(fa().fwd_split_workspace_bytes(1, 1, NL, D, True), dtype=torch.uint8,
                                 device=dev)}
    assert ws["fsplit"].numel() > 0  # the split path is the one captured

    def refill(seed):
        _fill(bufs, seed)
        bufs["qdec"].copy_(bufs["bf16"][0][:, :, N - NQ:])
        torch.cuda.synchronize()

    refill(11)
    eager = [t.clone() for t in _work(bufs, ws)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        _work(bufs, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _work(bufs, ws)

    for rep in range(3):
        # eager work between replays: another shape through the same library
        x = torch.randn(1, 2, 200, 64, device=dev).to(torch.bfloat16)
        fa().fwd(x, x, x, False)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(captured, eager)):
            assert torch.equal(got, want), f"replay {rep}: output {i} differs from the eager call"

    # the graph reads the captured input tensors' current contents
    refill(12)
    eager2 = [t.clone() for t in _work(bufs, ws)]
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(captured, eager2)):
        assert torch.equal(got, want), f"output {i} after refilling the inputs"
    assert not torch.equal(eager2[0], eager[0])

    # one head of the replayed bf16 results against the oracle
    q, k, v, do = (t[0, 1].double().cpu().numpy() for t in bufs["bf16"])
    o_ref, l_ref = oracle.attention_head_fwd64(q, k, v, True, SCALE)
    assert np.abs(captured[0][0, 1].double().cpu().numpy() - o_ref).max() <= 1e-2
    assert np.abs(captured[1][0, 1].double().cpu().numpy() - l_ref).max() <= 1e-3
    for got, ref in zip(captured[2:5], oracle.attention_head_bwd64(q, k, v, do, True, SCALE)):
        gg = got[0, 1].double().cpu().numpy()
        assert np.linalg.norm(gg - ref) / np.linalg.norm(ref) <= 2e-2
