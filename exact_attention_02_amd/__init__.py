"""MI355X (gfx950) exact attention: thin Python binding of libea02_attn.so.

The fused forward, its split-KV and decode form, the backward and absorbed
MLA decode.  The binding only marshals arguments: every step runs in the
library's HIP kernels.  PyTorch supplies device memory and the stream.  If
the library is not built, every call raises; there is no fallback path.

    out, lse = fwd(q, k, v, is_causal=True)          # allocates out and lse
    attn_fwd(q, k, v, out, lse, is_causal=True)      # caller-provided buffers
    out, lse = fwd_splitkv(q1, k, v, is_causal=True) # N_q != N_kv, key splits, decode
    dq, dk, dv = bwd(q, k, v, out, dout, lse, is_causal=True)   # backward

q: [B, H_q, N, D] bf16, k and v: [B, H_kv, N, D] bf16, contiguous, on the
current CUDA (HIP) device; out: like q; lse: [B, H_q, N] float32.  The split
entry points take q with N_q rows and k, v with N_kv rows.
The same names and semantics as the C functions declared in include/attn.h.
"""
from __future__ import annotations

import ctypes
import math
import os

from .build import LIB_PATH

__all__ = ["attn_fwd", "fwd", "attn_fwd_splitkv", "fwd_splitkv", "attn_splitkv_num_splits",
           "attn_fwd_splitkv_static", "attn_static_scratch_bytes",
           "attn_splitkv_workspace_size", "attn_bwd", "bwd", "attn_bwd_num_splits",
           "attn_bwd_workspace_size", "attention",
           "attn_mla_decode", "attn_mla_num_splits", "attn_mla_workspace_size", "mla_absorb_q",
           "mla_up_project", "mla_decode",
           "attn_status_string", "attn_abi_version",
           "load_library", "AttnError", "EXPORTED_SYMBOLS"]

EXPORTED_SYMBOLS = ("attn_fwd", "attn_fwd_splitkv", "attn_splitkv_num_splits",
                    "attn_fwd_splitkv_static", "attn_static_scratch_bytes",
                    "attn_splitkv_workspace_size", "attn_bwd", "attn_bwd_num_splits",
                    "attn_bwd_workspace_size",
                    "attn_mla_decode", "attn_mla_num_splits", "attn_mla_workspace_size",
                    "mla_absorb_q", "mla_up_project", "attn_status_string", "attn_abi_version")

_lib = None


class AttnError(RuntimeError):
    """A library entry point returned a nonzero status (see include/attn.h)."""

    def __init__(self, status: int, message: str, call: str = "libea02_attn"):
        super().__init__(f"{call} failed with status {status}: {message}")
        self.status = status
        self.call = call


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
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p]
    lib.attn_fwd_splitkv_static.restype = ctypes.c_int
    lib.attn_fwd_splitkv_static.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    lib.attn_static_scratch_bytes.restype = ctypes.c_size_t
    lib.attn_static_scratch_bytes.argtypes = []
    lib.attn_splitkv_num_splits.restype = ctypes.c_int64
    lib.attn_splitkv_num_splits.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int]
    lib.attn_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.attn_splitkv_workspace_size.argtypes = [ctypes.c_int64] * 5
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_bwd_num_splits.restype = ctypes.c_int64
    lib.attn_bwd_num_splits.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int64]
    lib.attn_mla_decode.restype = ctypes.c_int
    lib.attn_mla_decode.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p]
    lib.attn_mla_num_splits.restype = ctypes.c_int64
    lib.attn_mla_num_splits.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.attn_mla_workspace_size.restype = ctypes.c_size_t
    lib.attn_mla_workspace_size.argtypes = [ctypes.c_int64] * 4
    lib.mla_absorb_q.restype = ctypes.c_int
    lib.mla_absorb_q.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 6 + [ctypes.c_void_p]
    lib.mla_up_project.restype = ctypes.c_int
    lib.mla_up_project.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 5 + [ctypes.c_void_p]
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


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


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
    handle = _stream_handle(stream, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H_q, H_kv, N, D, float(sm_scale), int(bool(is_causal)), handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "attn_fwd")


def fwd(q, k, v, is_causal: bool = False, sm_scale: float | None = None, stream=None):
    """Allocate out [B,H_q,N,D] bf16 and lse [B,H_q,N] fp32, run attn_fwd, return both."""
    import torch
    B, H_q, N, D = q.shape
    out = torch.empty((B, H_q, N, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H_q, N), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, out, lse, is_causal=is_causal, sm_scale=sm_scale, stream=stream)
    return out, lse


def attn_splitkv_num_splits(B: int, H_q: int, H_kv: int, N_q: int, N_kv: int, D: int,
                            is_causal: bool = False) -> int:
    """Split count the library picks for n_splits=0 on the current device (-1: bad sizes)."""
    return int(load_library().attn_splitkv_num_splits(B, H_q, H_kv, N_q, N_kv, D,
                                                      int(bool(is_causal))))


def attn_splitkv_workspace_size(B: int, H_q: int, N_q: int, D: int, n_splits: int) -> int:
    """Workspace bytes attn_fwd_splitkv needs for n_splits key ranges (0 when n_splits <= 1)."""
    return int(load_library().attn_splitkv_workspace_size(B, H_q, N_q, D, n_splits))


def attn_fwd_splitkv(q, k, v, out, lse, is_causal: bool = False, sm_scale: float | None = None,
                     n_splits: int = 0, workspace=None, stream=None) -> None:
    """Enqueue the N_q x N_kv forward with n_splits key ranges (0: library's choice).

    workspace: a contiguous device tensor of at least attn_splitkv_workspace_size(...)
    bytes (any dtype), or None when the split count used is 1."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, H_q, N_q, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    _check_tensor(q, "q", (B, H_q, N_q, D), torch.bfloat16)
    _check_tensor(k, "k", (B, H_kv, N_kv, D), torch.bfloat16)
    _check_tensor(v, "v", (B, H_kv, N_kv, D), torch.bfloat16)
    _check_tensor(out, "out", (B, H_q, N_q, D), torch.bfloat16)
    _check_tensor(lse, "lse", (B, H_q, N_q), torch.float32)
    for name, t in (("k", k), ("v", v), ("out", out), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != q.device:
            raise ValueError("workspace must be a tensor on q's device")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), B, H_q, H_kv, N_q, N_kv, D, float(sm_scale),
                                  int(bool(is_causal)), int(n_splits), ws_ptr, ws_bytes, handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "attn_fwd_splitkv")


def attn_static_scratch_bytes() -> int:
    """Bytes of the library's static per-device scratch (attn_fwd_splitkv_static)."""
    return int(load_library().attn_static_scratch_bytes())


def attn_fwd_splitkv_static(q, k, v, out, lse, is_causal: bool = False,
                            sm_scale: float | None = None, n_splits: int = 0, stream=None) -> None:
    """attn_fwd_splitkv with its partial results in the library's static device
    scratch instead of a caller workspace: the call allocates nothing.  Calls
    that overlap on one GPU race on that scratch."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, H_q, N_q, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    _check_tensor(q, "q", (B, H_q, N_q, D), torch.bfloat16)
    _check_tensor(k, "k", (B, H_kv, N_kv, D), torch.bfloat16)
    _check_tensor(v, "v", (B, H_kv, N_kv, D), torch.bfloat16)
    _check_tensor(out, "out", (B, H_q, N_q, D), torch.bfloat16)
    _check_tensor(lse, "lse", (B, H_q, N_q), torch.float32)
    for name, t in (("k", k), ("v", v), ("out", out), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         lse.data_ptr(), B, H_q, H_kv, N_q, N_kv, D, float(sm_scale),
                                         int(bool(is_causal)), int(n_splits), handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "attn_fwd_splitkv_static")


def fwd_splitkv(q, k, v, is_causal: bool = False, sm_scale: float | None = None,
                n_splits: int = 0, stream=None):
    """Allocate out, lse and the workspace, run attn_fwd_splitkv, return (out, lse)."""
    import torch
    B, H_q, N_q, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    out = torch.empty((B, H_q, N_q, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        ns = n_splits if n_splits > 0 else attn_splitkv_num_splits(B, H_q, H_kv, N_q, N_kv, D,
                                                                   is_causal)
    ws = None
    if ns > 1:
        nbytes = attn_splitkv_workspace_size(B, H_q, N_q, D, ns)
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    attn_fwd_splitkv(q, k, v, out, lse, is_causal=is_causal, sm_scale=sm_scale,
                     n_splits=max(ns, 1), workspace=ws, stream=stream)
    return out, lse


def attn_bwd_num_splits(B: int, H_q: int, H_kv: int, N_q: int, N_kv: int, D: int,
                        is_causal: bool = False) -> int:
    """Row-range split count attn_bwd picks for n_splits=0 on the current device."""
    return int(load_library().attn_bwd_num_splits(B, H_q, H_kv, N_q, N_kv, D, int(bool(is_causal))))


def attn_bwd_workspace_size(B: int, H_q: int, H_kv: int, N_q: int, N_kv: int, D: int,
                            is_causal: bool = False, n_splits: int = 1) -> int:
    """Workspace bytes attn_bwd needs with n_splits dK/dV row ranges on the
    current device (per query row: log2-unit LSE and rowsum(dO*O); per range:
    fp32 partial dK and dV; fp32 partial dQ of the library's dQ splits)."""
    return int(load_library().attn_bwd_workspace_size(B, H_q, H_kv, N_q, N_kv, D,
                                                      int(bool(is_causal)), n_splits))


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, is_causal: bool = False,
             sm_scale: float | None = None, n_splits: int = 1, workspace=None,
             stream=None) -> None:
    """Enqueue the backward into dq, dk, dv (workspace: attn_bwd_workspace_size
    bytes for the split count used; n_splits=0 lets the library choose)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, H_q, N_q, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    for name, t, shape, dt in (("q", q, (B, H_q, N_q, D), torch.bfloat16),
                               ("k", k, (B, H_kv, N_kv, D), torch.bfloat16),
                               ("v", v, (B, H_kv, N_kv, D), torch.bfloat16),
                               ("out", out, (B, H_q, N_q, D), torch.bfloat16),
                               ("dout", dout, (B, H_q, N_q, D), torch.bfloat16),
                               ("lse", lse, (B, H_q, N_q), torch.float32),
                               ("dq", dq, (B, H_q, N_q, D), torch.bfloat16),
                               ("dk", dk, (B, H_kv, N_kv, D), torch.bfloat16),
                               ("dv", dv, (B, H_kv, N_kv, D), torch.bfloat16)):
        _check_tensor(t, name, shape, dt)
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != q.device:
            raise ValueError("workspace must be a tensor on q's device")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          B, H_q, H_kv, N_q, N_kv, D, float(sm_scale), int(bool(is_causal)),
                          int(n_splits), ws_ptr, ws_bytes, handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "attn_bwd")


def bwd(q, k, v, out, dout, lse, is_causal: bool = False, sm_scale: float | None = None,
        stream=None):
    """Allocate dq, dk, dv and the workspace, run attn_bwd with the library's
    split count, return (dq, dk, dv)."""
    import torch
    B, H_q, N_q, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    with torch.cuda.device(q.device):
        ns = max(attn_bwd_num_splits(B, H_q, H_kv, N_q, N_kv, D, is_causal), 1)
        nbytes = attn_bwd_workspace_size(B, H_q, H_kv, N_q, N_kv, D, is_causal, ns)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
    attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, is_causal=is_causal, sm_scale=sm_scale,
             n_splits=ns, workspace=ws, stream=stream)
    return dq, dk, dv


# ---------------------------------------------------------------- autograd
# The pages' autograd wrapper (page "Flash Attention 与 Kernel 优化", section
# "Autograd 包装与反向传播"): the forward saves q, k, v, O and the LSE, and
# the backward recomputes the probabilities from the LSE.  Here both passes
# are this library's entry points; the class only routes tensors.
_AUTOGRAD_FN = None


def _autograd_fn():
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is None:
        import torch

        class FlashAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, is_causal, sm_scale):
                if q.shape[2] == k.shape[2]:
                    out, lse = fwd(q, k, v, is_causal=is_causal, sm_scale=sm_scale)
                else:
                    out, lse = fwd_splitkv(q, k, v, is_causal=is_causal, sm_scale=sm_scale)
                ctx.save_for_backward(q, k, v, out, lse)
                ctx.is_causal, ctx.sm_scale = is_causal, sm_scale
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, out, lse = ctx.saved_tensors
                dq, dk, dv = bwd(q, k, v, out, dout.contiguous(), lse, is_causal=ctx.is_causal,
                                 sm_scale=ctx.sm_scale)
                return dq, dk, dv, None, None

        _AUTOGRAD_FN = FlashAttention
    return _AUTOGRAD_FN


def attention(q, k, v, is_causal: bool = False, sm_scale: float | None = None):
    """Differentiable attention: out = softmax(sm_scale q k^T [causal]) v with
    gradients for q, k and v (bf16, [B, H, N, D] contiguous on one device;
    N_q may differ from N_kv, causal then bottom-right aligned)."""
    return _autograd_fn().apply(q, k, v, bool(is_causal), sm_scale)


# ---------------------------------------------------------------- MLA decode
MLA_DC = 512
MLA_DR = 64


def attn_mla_num_splits(B: int, H: int, S: int, T: int, is_causal: bool = False) -> int:
    return int(load_library().attn_mla_num_splits(B, H, S, T, int(bool(is_causal))))


def attn_mla_workspace_size(B: int, H: int, S: int, n_splits: int) -> int:
    return int(load_library().attn_mla_workspace_size(B, H, S, n_splits))


def attn_mla_decode(q_lat, kv, out_lat, lse, sm_scale: float, is_causal: bool = False,
                    n_splits: int = 0, workspace=None, stream=None) -> None:
    """Latent attention core: q_lat [B,H,S,576], kv [B,T,576] -> out_lat [B,H,S,512], lse."""
    import torch
    if q_lat.dim() != 4 or kv.dim() != 3:
        raise ValueError("q_lat must be [B, H, S, 576] and kv [B, T, 576]")
    B, H, S, W = q_lat.shape
    T = kv.shape[1]
    _check_tensor(q_lat, "q_lat", (B, H, S, W), torch.bfloat16)
    _check_tensor(kv, "kv", (B, T, W), torch.bfloat16)
    _check_tensor(out_lat, "out_lat", (B, H, S, W - MLA_DR), torch.bfloat16)
    _check_tensor(lse, "lse", (B, H, S), torch.float32)
    for name, t in (("kv", kv), ("out_lat", out_lat), ("lse", lse)):
        if t.device != q_lat.device:
            raise ValueError(f"{name} is on {t.device}, q_lat on {q_lat.device}")
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != q_lat.device:
            raise ValueError("workspace must be a tensor on q_lat's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    handle = _stream_handle(stream, q_lat.device)
    with torch.cuda.device(q_lat.device):
        st = load_library().attn_mla_decode(q_lat.data_ptr(), kv.data_ptr(), out_lat.data_ptr(),
                                            lse.data_ptr(), B, H, S, T, W - MLA_DR, MLA_DR,
                                            float(sm_scale), int(bool(is_causal)), int(n_splits),
                                            ws_ptr, ws_bytes, handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "attn_mla_decode")


def mla_absorb_q(q_nope, q_pe, w_uk, q_lat, stream=None) -> None:
    """q_lat [B,H,S,576] = [q_nope W_uk[h], q_pe]; w_uk [H, d_nope, 512]."""
    import torch
    B, H, S, dn = q_nope.shape
    _check_tensor(q_nope, "q_nope", (B, H, S, dn), torch.bfloat16)
    _check_tensor(q_pe, "q_pe", (B, H, S, MLA_DR), torch.bfloat16)
    _check_tensor(w_uk, "w_uk", (H, dn, MLA_DC), torch.bfloat16)
    _check_tensor(q_lat, "q_lat", (B, H, S, MLA_DC + MLA_DR), torch.bfloat16)
    handle = _stream_handle(stream, q_nope.device)
    with torch.cuda.device(q_nope.device):
        st = load_library().mla_absorb_q(q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                                         q_lat.data_ptr(), B, H, S, dn, MLA_DC, MLA_DR, handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "mla_absorb_q")


def mla_up_project(out_lat, w_uv, out, stream=None) -> None:
    """out [B,H,S,d_v] = out_lat W_uv[h]^T; w_uv [H, d_v, 512]."""
    import torch
    B, H, S, dc = out_lat.shape
    d_v = w_uv.shape[1]
    _check_tensor(out_lat, "out_lat", (B, H, S, MLA_DC), torch.bfloat16)
    _check_tensor(w_uv, "w_uv", (H, d_v, MLA_DC), torch.bfloat16)
    _check_tensor(out, "out", (B, H, S, d_v), torch.bfloat16)
    handle = _stream_handle(stream, out_lat.device)
    with torch.cuda.device(out_lat.device):
        st = load_library().mla_up_project(out_lat.data_ptr(), w_uv.data_ptr(), out.data_ptr(),
                                           B, H, S, MLA_DC, d_v, handle)
    if st != 0:
        raise AttnError(st, attn_status_string(st), "mla_up_project")


def mla_decode(q_nope, q_pe, kv, w_uk, w_uv, sm_scale: float | None = None,
               is_causal: bool = False, n_splits: int = 0, stream=None):
    """Absorbed MLA decode: allocates the intermediates, returns (out [B,H,S,d_v], lse).

    kv is the latent cache [B, T, 576] = [c_kv, k_pe]; sm_scale defaults to
    1/sqrt(d_nope + 64)."""
    import torch
    B, H, S, dn = q_nope.shape
    T = kv.shape[1]
    dev = q_nope.device
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(dn + MLA_DR)
    q_lat = torch.empty((B, H, S, MLA_DC + MLA_DR), dtype=torch.bfloat16, device=dev)
    out_lat = torch.empty((B, H, S, MLA_DC), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    out = torch.empty((B, H, S, w_uv.shape[1]), dtype=torch.bfloat16, device=dev)
    with torch.cuda.device(dev):
        ns = n_splits if n_splits > 0 else attn_mla_num_splits(B, H, S, T, is_causal)
    nbytes = attn_mla_workspace_size(B, H, S, max(ns, 1))
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev) if nbytes else None
    mla_absorb_q(q_nope, q_pe, w_uk, q_lat, stream=stream)
    attn_mla_decode(q_lat, kv, out_lat, lse, sm_scale, is_causal=is_causal, n_splits=max(ns, 1),
                    workspace=ws, stream=stream)
    mla_up_project(out_lat, w_uv, out, stream=stream)
    return out, lse
