"""Python binding of libfa.so, the gfx950 exact-attention library (C ABI in include/fa.h).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.  PyTorch
supplies device memory (``torch.empty``) and the current HIP stream; tensors must be contiguous
[B, H, N, d] on a ROCm device.  There is no fallback: if the library is missing or a call fails, an
exception is raised.

Entry points (same names as the C ABI, without the ``fa_`` prefix):
  fwd(q, k, v, causal, scale=None) -> (o, lse)
  fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal, scale=None) -> (o, lse)
  bwd(q, k, v, o, lse, dout, causal, scale=None, workspace=None) -> (dq, dk, dv)
  bwd_workspace_bytes(B, H, N, d) -> int
  bwd_preprocess / bwd_dkdv / bwd_dq / bwd_delta_dq — the backward's phases (fa_bwd runs
      bwd_delta_dq, then bwd_dkdv), for scheduling or timing them apart
  bwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, dout, causal, scale=None,
          workspace=None) -> (dq, dk, dv)      (the backward of fwd_fp8)
  bwd_fp8_workspace_bytes(B, H, N, d) -> int
  status_str(code) -> str
  decode(q, k, v, causal, scale=None, workspace=None) -> (o, lse)   (q: [B,H,Nq,d], k/v: [B,H,Nk,d])
  decode_workspace_bytes(B, H, Nq, Nk, d) -> int
  device_info(device=0) -> (compute units, peak clock kHz), for pricing measurements
"""

import ctypes
import math
import os

import torch

__all__ = ["fwd", "fwd_split", "fwd_split_workspace_bytes", "fwd_fp8", "fwd_fp8_split", "bwd",
           "bwd_split",
           "bwd_split_workspace_bytes", "bwd_workspace_bytes", "bwd_preprocess", "bwd_dkdv",
           "bwd_dq", "bwd_delta_dq", "bwd_fp8", "bwd_fp8_workspace_bytes", "decode",
           "decode_workspace_bytes",
           "status_str", "device_info", "FaError", "library", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
_STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
           4: "FA_ERR_ALIGN", 5: "FA_ERR_WORKSPACE", 6: "FA_ERR_LAUNCH"}

_lib = None


class FaError(RuntimeError):
    """A libfa entry point returned a status other than FA_OK."""

    def __init__(self, fn, code, message):
        super().__init__(f"{fn} failed with status {code} ({message})")
        self.code = code


def library():
    """Load libfa.so (after torch, so it binds to the HIP runtime torch already loaded)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m io_aware_exact_18_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.fa_fwd.restype = i
        lib.fa_fwd_split_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.fa_fwd_split_workspace_bytes.restype = sz
        lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.fa_fwd_split.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, f, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_fwd_fp8_split.argtypes = [vp, vp, vp, f, f, f, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.fa_fwd_fp8_split.restype = i
        lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
        lib.fa_bwd_workspace_bytes.restype = sz
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_split_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.fa_bwd_split_workspace_bytes.restype = sz
        lib.fa_bwd_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f,
                                     vp]
        lib.fa_bwd_split.restype = i
        lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, sz, i, i, i, i, vp]
        lib.fa_bwd_preprocess.restype = i
        lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.fa_bwd_dkdv.restype = i
        lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.fa_bwd_delta_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.fa_bwd_delta_dq.restype = i
        lib.fa_bwd_dq.restype = i
        lib.fa_status_str.argtypes = [i]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_device_info.argtypes = [i, vp, vp]
        lib.fa_device_info.restype = i
        lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.fa_decode_workspace_bytes.restype = sz
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
        lib.fa_decode.restype = i
        lib.fa_bwd_fp8_workspace_bytes.argtypes = [i, i, i, i]
        lib.fa_bwd_fp8_workspace_bytes.restype = sz
        lib.fa_bwd_fp8.argtypes = ([vp, vp, vp, f, f, f] + [vp] * 7 + [sz, i, i, i, i, i, f, vp])
        lib.fa_bwd_fp8.restype = i
        _lib = lib
    return _lib


def device_info(device=0):
    """(compute units, peak shader clock in kHz) of a HIP device, from fa_device_info."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    _check("fa_device_info", library().fa_device_info(int(device), ctypes.byref(cus), ctypes.byref(khz)))
    return cus.value, khz.value


def status_str(code):
    return library().fa_status_str(int(code)).decode()


def _check(fn, code):
    if code != FA_OK:
        raise FaError(fn, code, status_str(code))


def _require(t, name, dtype, shape=None, device=None):
    """Checks one tensor argument: a contiguous ROCm tensor of this dtype (and shape, and the same
    device as the call's first tensor when ``device`` is given)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors are on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q, k, v, causal, scale=None):
    """Forward pass: returns (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    _require(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    _require(k, "k", torch.bfloat16, q.shape, device=q.device)
    _require(v, "v", torch.bfloat16, q.shape, device=q.device)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        code = library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, H, N, d, int(bool(causal)), _scale(scale, d),
                                _stream(q.device))
    _check("fa_fwd", code)
    return o, lse


def fwd_split_workspace_bytes(B, H, N, d, causal):
    """Bytes of workspace fa_fwd_split needs (0: the shape is not split, or is rejected)."""
    return int(library().fa_fwd_split_workspace_bytes(B, H, N, d, int(bool(causal))))


def fwd_split(q, k, v, causal, scale=None, workspace=None):
    """Forward pass that may split each query tile's key range (fa_fwd_split): returns (o, lse) as
    fwd.  The workspace (uint8, device) is allocated here when not given."""
    _require(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    _require(k, "k", torch.bfloat16, q.shape, device=q.device)
    _require(v, "v", torch.bfloat16, q.shape, device=q.device)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        ws_bytes = fwd_split_workspace_bytes(B, H, N, d, causal)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _require(workspace, "workspace", torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        code = library().fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H,
                                      N, d, int(bool(causal)), _scale(scale, d), _stream(q.device))
    _check("fa_fwd_split", code)
    return o, lse


def decode_workspace_bytes(B, H, Nq, Nk, d):
    """Bytes of workspace fa_decode needs (0 for a shape it rejects)."""
    return int(library().fa_decode_workspace_bytes(B, H, Nq, Nk, d))


def decode(q, k, v, causal, scale=None, workspace=None):
    """Decoding against a key/value cache: q [B,H,Nq,d] (1 ≤ Nq ≤ 32, the last Nq positions of the
    sequence), k and v [B,H,Nk,d] bf16.  Returns (o bf16 [B,H,Nq,d], lse fp32 [B,H,Nq])."""
    _require(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d]")
    B, H, Nq, d = q.shape
    _require(k, "k", torch.bfloat16, device=q.device)
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, {H}, Nk, {d}]")
    Nk = k.shape[2]
    _require(v, "v", torch.bfloat16, k.shape, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    ws_bytes = decode_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _require(workspace, "workspace", torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        code = library().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H,
                                   Nq, Nk, d, int(bool(causal)), _scale(scale, d), _stream(q.device))
    _check("fa_decode", code)
    return o, lse


def fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal, scale=None):
    """FP8 forward: e4m3fn codes with per-tensor descales in; (o bf16, lse fp32) out."""
    _require(q8, "q8", torch.float8_e4m3fn)
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    _require(k8, "k8", torch.float8_e4m3fn, q8.shape, device=q8.device)
    _require(v8, "v8", torch.float8_e4m3fn, q8.shape, device=q8.device)
    B, H, N, d = q8.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    with torch.cuda.device(q8.device):
        code = library().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), float(q_descale),
                                    float(k_descale), float(v_descale), o.data_ptr(),
                                    lse.data_ptr(), B, H, N, d, int(bool(causal)),
                                    _scale(scale, d), _stream(q8.device))
    _check("fa_fwd_fp8", code)
    return o, lse


def fwd_fp8_split(q8, k8, v8, q_descale, k_descale, v_descale, causal, scale=None, workspace=None):
    """FP8 forward that may split each query tile's key range (fa_fwd_fp8_split): returns (o, lse)
    as fwd_fp8.  The workspace (uint8, device) is allocated here when not given."""
    _require(q8, "q8", torch.float8_e4m3fn)
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    _require(k8, "k8", torch.float8_e4m3fn, q8.shape, device=q8.device)
    _require(v8, "v8", torch.float8_e4m3fn, q8.shape, device=q8.device)
    B, H, N, d = q8.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if workspace is None:
        workspace = torch.empty(max(fwd_split_workspace_bytes(B, H, N, d, causal), 256),
                                dtype=torch.uint8, device=q8.device)
    else:
        _require(workspace, "workspace", torch.uint8, device=q8.device)
    with torch.cuda.device(q8.device):
        code = library().fa_fwd_fp8_split(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(),
                                          float(q_descale), float(k_descale), float(v_descale),
                                          o.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), B, H, N, d, int(bool(causal)),
                                          _scale(scale, d), _stream(q8.device))
    _check("fa_fwd_fp8_split", code)
    return o, lse


def bwd_workspace_bytes(B, H, N, d):
    return int(library().fa_bwd_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, lse, dout, causal, scale=None, workspace=None):
    """Backward pass: returns (dq, dk, dv), bf16 [B,H,N,d].

    ``workspace`` is an optional preallocated uint8 device tensor of at least
    ``bwd_workspace_bytes(B, H, N, d)`` bytes; without it one is allocated per call.
    """
    _require(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _require(t, name, torch.bfloat16, q.shape, device=q.device)
    B, H, N, d = q.shape
    _require(lse, "lse", torch.float32, (B, H, N), device=q.device)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _require(workspace, "workspace", torch.uint8, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(q)
    dv = torch.empty_like(q)
    with torch.cuda.device(q.device):
        code = library().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H, N, d,
                                int(bool(causal)), _scale(scale, d), _stream(q.device))
    _check("fa_bwd", code)
    return dq, dk, dv


def bwd_split_workspace_bytes(B, H, N, d, causal):
    """Bytes of workspace fa_bwd_split needs (fa_bwd's when the shape is not split; 0 if rejected)."""
    return int(library().fa_bwd_split_workspace_bytes(B, H, N, d, int(bool(causal))))


def bwd_split(q, k, v, o, lse, dout, causal, scale=None, workspace=None):
    """Backward pass that may split the backward kernels' loops (fa_bwd_split): returns (dq, dk, dv)
    as bwd.  The workspace (uint8, device) is allocated here when not given."""
    _require(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _require(t, name, torch.bfloat16, q.shape, device=q.device)
    B, H, N, d = q.shape
    _require(lse, "lse", torch.float32, (B, H, N), device=q.device)
    if workspace is None:
        workspace = torch.empty(max(bwd_split_workspace_bytes(B, H, N, d, causal), 1),
                                dtype=torch.uint8, device=q.device)
    else:
        _require(workspace, "workspace", torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    with torch.cuda.device(q.device):
        code = library().fa_bwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                      dv.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H,
                                      N, d, int(bool(causal)), _scale(scale, d), _stream(q.device))
    _check("fa_bwd_split", code)
    return dq, dk, dv


def bwd_fp8_workspace_bytes(B, H, N, d):
    return int(library().fa_bwd_fp8_workspace_bytes(B, H, N, d))


def bwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, dout, causal, scale=None,
            workspace=None):
    """Backward of the FP8 forward: e4m3fn codes with their descales, fwd_fp8's (o, lse) and a bf16
    upstream gradient in; (dq, dk, dv) bf16 out, the gradients with respect to the dequantised
    inputs.  ``workspace``: optional uint8 device tensor of ``bwd_fp8_workspace_bytes`` bytes."""
    _require(q8, "q8", torch.float8_e4m3fn)
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    _require(k8, "k8", torch.float8_e4m3fn, q8.shape, device=q8.device)
    _require(v8, "v8", torch.float8_e4m3fn, q8.shape, device=q8.device)
    _require(o, "o", torch.bfloat16, q8.shape, device=q8.device)
    _require(dout, "dout", torch.bfloat16, q8.shape, device=q8.device)
    B, H, N, d = q8.shape
    _require(lse, "lse", torch.float32, (B, H, N), device=q8.device)
    need = bwd_fp8_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q8.device)
    else:
        _require(workspace, "workspace", torch.uint8, device=q8.device)
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
                  for _ in range(3))
    with torch.cuda.device(q8.device):
        code = library().fa_bwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), float(q_descale),
                                    float(k_descale), float(v_descale), o.data_ptr(),
                                    lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H,
                                    N, d, int(bool(causal)), _scale(scale, d), _stream(q8.device))
    _check("fa_bwd_fp8", code)
    return dq, dk, dv


def bwd_preprocess(o, dout, workspace):
    """Phase 1 of the backward: D = rowsum(dO ∘ O) into ``workspace``."""
    _require(o, "o", torch.bfloat16)
    _require(dout, "dout", torch.bfloat16, o.shape, device=o.device)
    _require(workspace, "workspace", torch.uint8, device=o.device)
    B, H, N, d = o.shape
    with torch.cuda.device(o.device):
        code = library().fa_bwd_preprocess(o.data_ptr(), dout.data_ptr(), workspace.data_ptr(),
                                           workspace.numel(), B, H, N, d, _stream(o.device))
    _check("fa_bwd_preprocess", code)


def _bwd_inputs(q, k, v, lse, dout, workspace, outs):
    _require(q, "q", torch.bfloat16)
    for t, name in ((k, "k"), (v, "v"), (dout, "dout"), *outs):
        _require(t, name, torch.bfloat16, q.shape, device=q.device)
    B, H, N, d = q.shape
    _require(lse, "lse", torch.float32, (B, H, N), device=q.device)
    _require(workspace, "workspace", torch.uint8, device=q.device)
    return B, H, N, d


def bwd_dkdv(q, k, v, lse, dout, dk, dv, workspace, causal, scale=None):
    """Phase 2 of the backward: writes dk and dv (needs bwd_preprocess on the same workspace)."""
    B, H, N, d = _bwd_inputs(q, k, v, lse, dout, workspace, ((dk, "dk"), (dv, "dv")))
    with torch.cuda.device(q.device):
        code = library().fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                                     dout.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), B, H, N, d,
                                     int(bool(causal)), _scale(scale, d), _stream(q.device))
    _check("fa_bwd_dkdv", code)


def bwd_dq(q, k, v, lse, dout, dq, workspace, causal, scale=None):
    """Phase 3 of the backward: writes dq (needs bwd_preprocess on the same workspace)."""
    B, H, N, d = _bwd_inputs(q, k, v, lse, dout, workspace, ((dq, "dq"),))
    with torch.cuda.device(q.device):
        code = library().fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                                   dout.data_ptr(), dq.data_ptr(), workspace.data_ptr(),
                                   workspace.numel(), B, H, N, d, int(bool(causal)),
                                   _scale(scale, d), _stream(q.device))
    _check("fa_bwd_dq", code)


def bwd_delta_dq(q, k, v, o, lse, dout, dq, workspace, causal, scale=None):
    """D into the workspace and dq in one phase (what bwd_preprocess then bwd_dq give, bit for bit);
    bwd_dkdv on the same workspace may follow."""
    B, H, N, d = _bwd_inputs(q, k, v, lse, dout, workspace, ((o, "o"), (dq, "dq")))
    with torch.cuda.device(q.device):
        code = library().fa_bwd_delta_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), B, H, N, d,
                                         int(bool(causal)), _scale(scale, d), _stream(q.device))
    _check("fa_bwd_delta_dq", code)
