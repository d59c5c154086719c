"""fa_bwd_noalloc (the backward with its workspace in the library's fixed device array) against
fa_bwd with a caller-allocated workspace: the same kernels, so the gradients must agree bit for bit.
Two calls in a row, the second on a smaller input, so stale contents of the shared array from the
first call cannot hide a missing write."""

import ctypes
import math

import pytest
import torch

pytestmark = pytest.mark.gpu


def _lib():
    import io_aware_exact_18_amd as fa
    lib = fa.library()
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, i, f, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_max_rows.argtypes = []
    lib.fa_bwd_noalloc_max_rows.restype = ctypes.c_size_t
    return lib


def _case(B, H, N, d, causal, seed):
    import io_aware_exact_18_amd as fa
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v, do = (torch.randn(B, H, N, d, generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd(q, k, v, causal, scale)
    want = fa.bwd(q, k, v, o, lse, do, causal, scale)
    got = [torch.empty_like(q) for _ in range(3)]
    code = _lib().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), do.data_ptr(), got[0].data_ptr(), got[1].data_ptr(),
                                 got[2].data_ptr(), B, H, N, d, int(causal), scale,
                                 torch.cuda.current_stream().cuda_stream)
    assert code == 0, code
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("d", [64, 128])
def test_noalloc_matches_fa_bwd_twice(d):
    assert torch.cuda.is_available()
    for (B, H, N, causal, seed) in ((2, 4, 1000, True, 1), (1, 3, 321, False, 2)):
        got, want = _case(B, H, N, d, causal, seed + d)
        for a, b in zip(got, want):
            assert torch.equal(a, b), (B, H, N, d, causal)


def test_noalloc_largest_and_rejected_shapes():
    """B·H·N = 2^22 rows (the array's capacity) works and matches fa_bwd; one row more is refused
    with FA_ERR_WORKSPACE before anything is enqueued."""
    lib = _lib()
    assert lib.fa_bwd_noalloc_max_rows() == 1 << 22
    got, want = _case(1, 1024, 4096, 64, True, 3)
    for a, b in zip(got, want):
        assert torch.equal(a, b)
    p = 1 << 12
    assert lib.fa_bwd_noalloc(*([p] * 9), 1, 1, (1 << 22) + 1, 64, 1, 0.125, None) == 5
