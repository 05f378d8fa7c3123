"""MI355X (gfx950) fused attention forward: thin Python binding of libea02_attn.so.

The binding only marshals arguments: every step of the attention forward runs
in the library's HIP kernels.  PyTorch supplies device memory and the stream.
If the library is not built, every call raises; there is no fallback path.

    out, lse = fwd(q, k, v, is_causal=True)          # allocates out and lse
    attn_fwd(q, k, v, out, lse, is_causal=True)      # caller-provided buffers

q: [B, H_q, N, D] bf16, k and v: [B, H_kv, N, D] bf16, contiguous, on the
current CUDA (HIP) device; out: like q; lse: [B, H_q, N] float32.
The same names and semantics as the C functions declared in include/attn.h.
"""
from __future__ import annotations

import ctypes
import math
import os

from .build import LIB_PATH

__all__ = ["attn_fwd", "fwd", "attn_status_string", "attn_abi_version", "load_library",
           "AttnError", "EXPORTED_SYMBOLS"]

EXPORTED_SYMBOLS = ("attn_fwd", "attn_status_string", "attn_abi_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attn_fwd failed with status {status}: {message}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m exact_attention_02_amd.build`")
    lib = ctypes.CDLL(p)
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_abi_version.restype = ctypes.c_int
    lib.attn_abi_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_abi_version() -> int:
    return int(load_library().attn_abi_version())


def _check_tensor(t, name, shape, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_fwd(q, k, v, out, lse, is_causal: bool = False, sm_scale: float | None = None,
             stream=None) -> None:
    """Enqueue the forward on `stream` (default: torch's current stream) into out/lse."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, H_q, N, D = q.shape
    H_kv = k.shape[1]
    _check_tensor(q, "q", (B, H_q, N, D), torch.bfloat16)
    _check_tensor(k, "k", (B, H_kv, N, D), torch.bfloat16)
    _check_tensor(v, "v", (B, H_kv, N, D), torch.bfloat16)
    _check_tensor(out, "out", (B, H_q, N, D), torch.bfloat16)
    _check_tensor(lse, "lse", (B, H_q, N), torch.float32)
    for name, t in (("k", k), ("v", v), ("out", out), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H_q, H_kv, N, D, float(sm_scale), int(bool(is_causal)), handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st))


def fwd(q, k, v, is_causal: bool = False, sm_scale: float | None = None, stream=None):
    """Allocate out [B,H_q,N,D] bf16 and lse [B,H_q,N] fp32, run attn_fwd, return both."""
    import torch
    B, H_q, N, D = q.shape
    out = torch.empty((B, H_q, N, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H_q, N), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, out, lse, is_causal=is_causal, sm_scale=sm_scale, stream=stream)
    return out, lse
