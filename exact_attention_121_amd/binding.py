"""Thin Python binding of libattn_fwd.so (argument marshalling only).

Every step of the attention forward runs in the HIP kernels behind the C ABI
declared in include/attn_fwd.h.  This module only checks tensor metadata,
allocates outputs with torch (device memory), passes raw pointers and torch's
current HIP stream, and turns status codes into exceptions.  There is no
fallback: if the library is missing or the tensors are not on an AMD GPU, the
call fails loudly.
"""

from __future__ import annotations

import ctypes
import math
import os

from .build import LIB_PATH

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_DEVICE = 3
ATTN_ERR_SCRATCH = 4
BWD_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ("attn_fwd", "attn_fwd_bf16", "attn_check_args", "attn_decode", "attn_decode_bf16", "attn_decode_workspace_size",
           "attn_check_decode_args", "attn_bwd", "attn_bwd_bf16", "attn_bwd_workspace_size", "attn_check_bwd_args", "attn_bwd_noalloc",
           "attn_status_string", "attn_version")

_lib = None


class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"attn status {status}: {message}")
        self.status = status


class AttnUnsupportedError(AttnError, NotImplementedError):
    """head_dim not a multiple of 32 in [32, 256]; the caller may use an unfused path."""


class AttnArgumentError(AttnError, ValueError):
    """Invalid argument (see attn_check_args)."""


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libattn_fwd.so once and declare its signatures.  With a path, that
    build of the library (e.g. a variant from build.variant_path) is loaded
    and returned instead, without replacing the default one.  The environment
    variable ATTN_LIBRARY names another default build (the CPU tests use it to
    run against a sanitizer build of the host code)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("ATTN_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m exact_attention_121_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    # PyTorch ships its own HIP runtime and asks for it under another file
    # name than this library does (libamdhip64.so against libamdhip64.so.7,
    # one soname).  Loaded first, torch's copy also satisfies this library;
    # loaded after it, torch would bring a second runtime, whose streams this
    # library's launches would then reject.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                             ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_bf16.argtypes = lib.attn_fwd.argtypes
    lib.attn_fwd_bf16.restype = ctypes.c_int
    lib.attn_check_args.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float]
    lib.attn_check_args.restype = ctypes.c_int
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                ctypes.c_int, vp, i64, vp]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_bf16.argtypes = lib.attn_decode.argtypes
    lib.attn_decode_bf16.restype = ctypes.c_int
    lib.attn_decode_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.attn_decode_workspace_size.restype = ctypes.c_int
    lib.attn_check_decode_args.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                           ctypes.c_float, vp, i64]
    lib.attn_check_decode_args.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                             ctypes.c_int, vp, i64, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_bf16.argtypes = lib.attn_bwd.argtypes
    lib.attn_bwd_bf16.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.attn_bwd_workspace_size.restype = ctypes.c_int
    lib.attn_check_bwd_args.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                        ctypes.c_float, vp, i64]
    lib.attn_check_bwd_args.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                     ctypes.c_int, vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_version() -> str:
    return load_library().attn_version().decode()


def attn_check_args(q, k, v, o, lse, B, Hq, Hkv, N, d, scale) -> int:
    """Host-only validation (pointers as integers or None); returns a status."""
    return load_library().attn_check_args(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale))


def _raise_for(status: int):
    if status == ATTN_OK:
        return
    msg = attn_status_string(status)
    if status == ATTN_ERR_UNSUPPORTED:
        raise AttnUnsupportedError(status, msg)
    if status == ATTN_ERR_INVALID_ARG:
        raise AttnArgumentError(status, msg)
    raise AttnError(status, msg)


def _keep_for_stream(s, *tensors):
    """Marks tensors this module allocated on the current stream as used by
    stream ``s`` when the kernels run there: torch's caching allocator then
    waits for the work queued on ``s`` before it hands their memory to another
    allocation (the decode partials and the backward's per-row terms are
    written by one kernel and read by a later one, after the call returns)."""
    import torch

    if s == torch.cuda.current_stream(s.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def attn_fwd(q, k, v, *, scale: float | None = None, causal: bool = False, out=None,
             lse=None, return_lse: bool = True, stream=None, library=None):
    """Fused attention forward on torch fp16 or bf16 tensors resident on one AMD GPU.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; contiguous torch.float16 (or all
    torch.bfloat16) on the same HIP device; o has the same type.  scale defaults to 1/sqrt(d).  Returns (o, lse) with o
    [B, Hq, N, d] fp16 and lse [B, Hq, N] fp32 (None if return_lse is False
    and no lse buffer is given).  The kernel is queued on ``stream`` (a
    torch.cuda.Stream) or on torch's current stream of q's device.
    ``library``: a library handle from load_library(path) to call instead of
    the default build.
    """
    import torch

    if not isinstance(q, torch.Tensor) or q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("q must be a torch.float16 or torch.bfloat16 tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on an AMD GPU (torch 'cuda' device), got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    made = []
    if out is None:
        out = torch.empty_like(q)
        made.append(out)
    elif (out.shape != q.shape or out.dtype != q.dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor of q's dtype, shaped like q on q's device")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        made.append(lse)
    elif lse is not None and (lse.shape != (B, Hq, N) or lse.dtype != torch.float32
                              or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 tensor [B, Hq, N] on q's device")

    lib = library if library is not None else load_library()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        _keep_for_stream(s, *made)
        fn = lib.attn_fwd_bf16 if q.dtype == torch.bfloat16 else lib.attn_fwd
        status = fn(
            q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
            out.data_ptr() or None, (lse.data_ptr() or None) if lse is not None else None,
            B, Hq, Hkv, N, d, float(scale), 1 if causal else 0, s.cuda_stream or None)
    _raise_for(status)
    return out, lse


def attn_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d) -> int:
    """Workspace bytes attn_decode needs for this shape (host only)."""
    out = ctypes.c_int64(0)
    _raise_for(load_library().attn_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, ctypes.byref(out)))
    return out.value


def attn_check_decode_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, workspace, workspace_bytes) -> int:
    """Host-only validation of attn_decode (pointers as integers or None); returns a status."""
    return load_library().attn_check_decode_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale),
                                                 workspace, workspace_bytes)


def attn_decode(q, k, v, *, scale: float | None = None, causal: bool = True, out=None, lse=None,
                return_lse: bool = True, workspace=None, stream=None, library=None):
    """Decode step on torch fp16 (or bf16) tensors: q [B, Hq, Nq, d] are the last Nq
    positions of a sequence whose keys/values k, v [B, Hkv, Nk, d] are
    cached (Nq <= Nk).  With causal, query i sees keys 0 .. Nk - Nq + i.
    ``workspace`` is an optional uint8 device tensor of at least
    attn_decode_workspace_size(...) bytes (allocated here when omitted).
    Returns (o, lse) like attn_fwd.
    """
    import torch

    if not isinstance(q, torch.Tensor) or q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("q must be a torch.float16 or torch.bfloat16 tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on an AMD GPU (torch 'cuda' device), got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, Hq, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    made = []
    if out is None:
        out = torch.empty_like(q)
        made.append(out)
    elif (out.shape != q.shape or out.dtype != q.dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor of q's dtype, shaped like q on q's device")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
        made.append(lse)
    elif lse is not None and (lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32
                              or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 tensor [B, Hq, Nq] on q's device")
    need = attn_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()

    lib = library if library is not None else load_library()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        _keep_for_stream(s, *made)
        fn = lib.attn_decode_bf16 if q.dtype == torch.bfloat16 else lib.attn_decode
        status = fn(
            q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
            out.data_ptr() or None, (lse.data_ptr() or None) if lse is not None else None,
            B, Hq, Hkv, Nq, Nk, d, float(scale), 1 if causal else 0,
            workspace.data_ptr() or None, ws_bytes, s.cuda_stream or None)
    _raise_for(status)
    return out, lse


def attn_bwd_workspace_size(B, Hq, N, d) -> int:
    """Workspace bytes attn_bwd needs for this shape (host only)."""
    out = ctypes.c_int64(0)
    _raise_for(load_library().attn_bwd_workspace_size(B, Hq, N, d, ctypes.byref(out)))
    return out.value


def attn_check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, workspace,
                        workspace_bytes) -> int:
    """Host-only validation of attn_bwd (pointers as integers or None); returns a status."""
    return load_library().attn_check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d,
                                              float(scale), workspace, workspace_bytes)


def attn_bwd(q, k, v, o, lse, dout, *, scale: float | None = None, causal: bool = False, dq=None, dk=None,
             dv=None, workspace=None, stream=None, library=None):
    """Attention backward on torch tensors resident on one AMD GPU.

    q, o, dout: [B, Hq, N, d] and k, v: [B, Hkv, N, d], all fp16 or all bf16, with o and
    lse ([B, Hq, N] fp32) as attn_fwd returned them for the same q, k, v,
    scale and causal.  Returns (dq, dk, dv) shaped like q, k, v.
    ``workspace`` is an optional uint8 device tensor of at least
    attn_bwd_workspace_size(...) bytes (allocated here when omitted).
    """
    import torch

    if not isinstance(q, torch.Tensor) or q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("q must be a torch.float16 or torch.bfloat16 tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on an AMD GPU (torch 'cuda' device), got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("all tensors must be on q's device")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, Hq, N) or lse.dtype != torch.float32
            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be the contiguous fp32 [B, Hq, N] tensor attn_fwd returned")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs, made = [], []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
            made.append(t)
        elif (t.shape != like.shape or t.dtype != q.dtype or t.device != q.device
              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor of q's dtype shaped like its input")
        outs.append(t)
    dq, dk, dv = outs
    need = attn_bwd_workspace_size(B, Hq, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()

    lib = library if library is not None else load_library()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        _keep_for_stream(s, *made)
        fn = lib.attn_bwd_bf16 if q.dtype == torch.bfloat16 else lib.attn_bwd
        status = fn(
            q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
            lse.data_ptr() or None, dout.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
            dv.data_ptr() or None, B, Hq, Hkv, N, d, float(scale), 1 if causal else 0,
            workspace.data_ptr() or None, ws_bytes, s.cuda_stream or None)
    _raise_for(status)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, *, scale: float | None = None, causal: bool = False,
                     stream=None):
    """attn_bwd for fp16 tensors with the library's fixed scratch instead of a
    workspace: neither this wrapper nor the library allocates anything, so the
    outputs dq, dk, dv must be given.  For problems with B * Hq * round_up(N,
    128) <= 2^21; larger ones raise (ATTN_ERR_SCRATCH).  Calls in flight at
    once on one GPU share its scratch and must not overlap.
    Returns (dq, dk, dv)."""
    import torch

    ts = (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv))
    for name, t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be torch.float16, got {t.dtype}")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError(f"{name} must be on q's AMD GPU (torch 'cuda' device), got {t.device}")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D [B, H, N, d] tensor")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o.shape != q.shape or dout.shape != q.shape or dq.shape != q.shape:
        raise ValueError("o, dout and dq must be shaped like q")
    if dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("dk and dv must be shaped like k")
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, Hq, N) or lse.dtype != torch.float32
            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be the contiguous fp32 [B, Hq, N] tensor attn_fwd returned")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load_library()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = lib.attn_bwd_noalloc(
            q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
            lse.data_ptr() or None, dout.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
            dv.data_ptr() or None, B, Hq, k.shape[1], N, d, float(scale), 1 if causal else 0, s.cuda_stream or None)
    _raise_for(status)
    return dq, dk, dv
