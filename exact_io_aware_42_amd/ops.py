"""Thin Python binding of libfa2.so (ctypes): argument marshalling only.

Every step of the attention computation runs in the HIP kernels behind the C ABI declared in
include/fa2.h. PyTorch supplies device memory and the current stream; nothing here computes
attention, and there is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

# The in-tree library; FA2_LIBRARY may name another build of the same sources.
LIB_PATH = os.environ.get("FA2_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfa2.so")

FA2_OK = 0
FA2_ERR_INVALID_ARGUMENT = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_HIP = 3
FA2_ERR_SCRATCH_LIMIT = 4

EXPORTED = ("fa2_fwd", "fa2_bwd", "fa2_bwd_workspace_bytes", "fa2_bwd_preprocess",
            "fa2_bwd_dkdv", "fa2_bwd_dq", "fa2_fwd_gqa", "fa2_bwd_gqa", "fa2_fwd_dropout",
            "fa2_bwd_dropout", "fa2_bwd_gqa_workspace_bytes", "fa2_bwd_noalloc",
            "fa2_bwd_noalloc_max_rows", "fa2_status_string", "fa2_last_hip_error")

_lib = None
_lock = threading.Lock()


class FA2Error(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa2.so once and declare its signatures. Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = open_library(path)
        return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A new handle on a build of the library at `path` (e.g. the FA2_DEBUG_SYNC build), with
    its signatures declared; not cached. Raises if the file is missing."""
    if not os.path.exists(path):
        raise FA2Error(f"{path} is missing: build it with "
                       "`python -m exact_io_aware_42_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    ll, ull = ctypes.c_longlong, ctypes.c_ulonglong
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa2_fwd.restype = i
    lib.fa2_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                            i, i, i, i, i, f, vp]
    lib.fa2_bwd.restype = i
    lib.fa2_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, vp]
    lib.fa2_bwd_preprocess.restype = i
    lib.fa2_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, f, vp]
    lib.fa2_bwd_dkdv.restype = i
    lib.fa2_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, f, vp]
    lib.fa2_bwd_dq.restype = i
    lib.fa2_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ll, i, f, vp]
    lib.fa2_fwd_gqa.restype = i
    lib.fa2_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                i, i, i, i, i, ll, i, f, vp]
    lib.fa2_bwd_gqa.restype = i
    lib.fa2_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ll, i, f, f, ull, ull,
                                    vp]
    lib.fa2_fwd_dropout.restype = i
    lib.fa2_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                    i, i, i, i, i, ll, i, f, f, ull, ull, vp]
    lib.fa2_bwd_dropout.restype = i
    lib.fa2_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa2_bwd_workspace_bytes.restype = sz
    lib.fa2_bwd_gqa_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa2_bwd_gqa_workspace_bytes.restype = sz
    lib.fa2_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa2_bwd_noalloc.restype = i
    lib.fa2_bwd_noalloc_max_rows.argtypes = []
    lib.fa2_bwd_noalloc_max_rows.restype = sz
    lib.fa2_status_string.argtypes = [i]
    lib.fa2_status_string.restype = ctypes.c_char_p
    lib.fa2_last_hip_error.argtypes = []
    lib.fa2_last_hip_error.restype = i
    return lib


def _check(status: int, what: str):
    if status != FA2_OK:
        lib = load_library()
        name = lib.fa2_status_string(status).decode()
        extra = f" (HIP error {lib.fa2_last_hip_error()})" if status == FA2_ERR_HIP else ""
        raise FA2Error(f"{what} failed: {name}{extra}")


def _check_tensor(t: torch.Tensor, name: str, shape, dtype=torch.bfloat16, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device) -> int:
    """The current torch stream of `device`. The library launches on the calling thread's
    current HIP device, so the tensors' device must be the current one."""
    if device.index is not None and device.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {device} but the current device is "
                         f"cuda:{torch.cuda.current_device()}; call under "
                         f"torch.cuda.device({device.index})")
    return torch.cuda.current_stream(device).cuda_stream


def _ws_check(workspace, device, need: int):
    """Pointer and size of a workspace: a contiguous buffer on `device` of >= `need` bytes."""
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError(f"workspace must be a tensor on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace has {nbytes} bytes, needs at least {need}")
    return workspace.data_ptr(), nbytes


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def _u64(x: int) -> int:
    return int(x) & 0xFFFFFFFFFFFFFFFF


def _kv_layout(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    """(Hkv, batch stride in elements) of k and v: [B, Hkv, N, d] with heads, rows and columns
    contiguous, the same strides for both (separate tensors, or views of a packed
    [B, 2, Hkv, N, d] tensor); H must be a multiple of Hkv."""
    B, H, N, d = q.shape
    for t, nm in ((k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{nm} must be a [B, Hkv, N, d] tensor")
        if t.device != q.device or t.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bfloat16 on {q.device}")
    if q.numel() == 0:  # empty problem: nothing is read (the library returns at once)
        return H, H * N * d
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError(f"k, v must be [B, Hkv, N, d] = [{B}, Hkv, {N}, {d}]")
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"the {H} query heads must be a multiple of the {Hkv} K/V heads")
    # strides of size-1 dimensions do not address anything and are not compared
    inner = (N * d, d, 1)
    for t in (k, v):
        if any(t.shape[i + 1] > 1 and t.stride(i + 1) != inner[i] for i in range(3)):
            raise ValueError("k and v need contiguous heads, rows and columns")
    if B > 1 and k.stride(0) != v.stride(0):
        raise ValueError("k and v need equal batch strides")
    kvs = k.stride(0) if B > 1 else Hkv * N * d
    return Hkv, kvs


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: float | None = None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, dropout_p: float = 0.0, seed: int = 0,
        offset: int = 0):
    """Attention forward on bf16 [B, H, N, d] tensors. Returns (o bf16, lse fp32 [B, H, N]).
    k and v may have fewer heads (Hkv dividing H: grouped heads) and may be views of one packed
    [B, 2, Hkv, N, d] tensor. dropout_p > 0 drops probabilities with the counter-based mask of
    (seed, offset) declared in include/fa2.h; bwd must get the same three values."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    _check_tensor(q, "q", (B, H, N, d), device=dev)
    Hkv, kvs = _kv_layout(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", (B, H, N, d), device=dev)
    _check_tensor(lse, "lse", (B, H, N), dtype=torch.float32, device=dev)
    s = default_scale(d) if scale is None else float(scale)
    if dropout_p:
        st = lib.fa2_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, H, Hkv, N, d, kvs, int(bool(causal)), s,
                                 float(dropout_p), _u64(seed), _u64(offset), _stream_ptr(dev))
    elif Hkv == H and kvs == H * N * d:
        st = lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), B, H, N, d, int(bool(causal)), s, _stream_ptr(dev))
    else:
        st = lib.fa2_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, Hkv, N, d, kvs, int(bool(causal)), s,
                             _stream_ptr(dev))
    _check(st, "fa2_fwd")
    return out, lse


def fwd_kvpacked(q: torch.Tensor, kv: torch.Tensor, causal: bool = False,
                 scale: float | None = None):
    """Forward with K and V packed in one contiguous bf16 [B, 2, Hkv, N, d] tensor."""
    if kv.dim() != 5 or kv.shape[1] != 2 or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [B, 2, Hkv, N, d] tensor")
    return fwd(q, kv[:, 0], kv[:, 1], causal=causal, scale=scale)


def bwd_workspace_bytes(B: int, H: int, N: int, d: int, Hkv: int | None = None) -> int:
    """Backward workspace bytes: the minimum (fa2_bwd_workspace_bytes), or with Hkv given the
    size that lets small problems split their dK/dV work (fa2_bwd_gqa_workspace_bytes)."""
    lib = load_library()
    if Hkv is None:
        return int(lib.fa2_bwd_workspace_bytes(B, H, N, d))
    return int(lib.fa2_bwd_gqa_workspace_bytes(B, H, Hkv, N, d))


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, workspace=None, dropout_p: float = 0.0, seed: int = 0,
        offset: int = 0):
    """Attention backward. Returns (dq, dk, dv) bf16; dk, dv have k's and v's layout (grouped
    and packed K/V as in fwd); dropout arguments as given to fwd."""
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    for t, nm in ((q, "q"), (o, "o"), (dout, "dout")):
        _check_tensor(t, nm, (B, H, N, d), device=dev)
    Hkv, kvs = _kv_layout(q, k, v)
    _check_tensor(lse, "lse", (B, H, N), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    _check_tensor(dq, "dq", (B, H, N, d), device=dev)
    if dk is None:
        dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=dev)
    if dv is None:
        dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=dev)
    if _kv_layout(q, dk, dv) != (Hkv, kvs):
        raise ValueError("dk and dv must have the layout of k and v")
    if workspace is None:
        full = bwd_workspace_bytes(B, H, N, d, Hkv)
        workspace = torch.empty(max(full, 1), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _ws_check(workspace, dev, bwd_workspace_bytes(B, H, N, d))
    s = default_scale(d) if scale is None else float(scale)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_bytes)
    if dropout_p:
        st = lib.fa2_bwd_dropout(*ptrs, B, H, Hkv, N, d, kvs, int(bool(causal)), s,
                                 float(dropout_p), _u64(seed), _u64(offset), _stream_ptr(dev))
    elif Hkv == H and kvs == H * N * d:
        st = lib.fa2_bwd(*ptrs, B, H, N, d, int(bool(causal)), s, _stream_ptr(dev))
    else:
        st = lib.fa2_bwd_gqa(*ptrs, B, H, Hkv, N, d, kvs, int(bool(causal)), s,
                             _stream_ptr(dev))
    _check(st, "fa2_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool = False,
                scale: float | None = None):
    """Backward into caller-given dq, dk, dv with the library's static scratch in place of a
    workspace (fa2_bwd_noalloc: nothing is allocated, here or in the library). Same results
    as bwd with the minimum workspace; B*H*N at most fa2_bwd_noalloc_max_rows()."""
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"),
                  (dk, "dk"), (dv, "dv")):
        _check_tensor(t, nm, (B, H, N, d), device=dev)
    _check_tensor(lse, "lse", (B, H, N), dtype=torch.float32, device=dev)
    s = default_scale(d) if scale is None else float(scale)
    st = lib.fa2_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), B, H, N, d, int(bool(causal)), s, _stream_ptr(dev))
    _check(st, "fa2_bwd_noalloc")
    return dq, dk, dv


def bwd_noalloc_max_rows() -> int:
    return int(load_library().fa2_bwd_noalloc_max_rows())


def bwd_kvpacked(q, kv, o, dout, lse, causal: bool = False, scale: float | None = None):
    """Backward for packed K/V: returns (dq, dkv) with dkv [B, 2, Hkv, N, d] like kv."""
    if kv.dim() != 5 or kv.shape[1] != 2 or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [B, 2, Hkv, N, d] tensor")
    dkv = torch.empty_like(kv)
    dq, _, _ = bwd(q, kv[:, 0], kv[:, 1], o, dout, lse, causal=causal, scale=scale,
                   dk=dkv[:, 0], dv=dkv[:, 1])
    return dq, dkv


def _ws(workspace: torch.Tensor, device, B: int, H: int, N: int, d: int):
    return _ws_check(workspace, device, bwd_workspace_bytes(B, H, N, d))


def bwd_preprocess(o, dout, lse, workspace):
    """Fill `workspace` with -D, D = rowsum(dout * o), and LSE * log2(e) (bwd_dq does this too;
    this stage is for callers that need dK/dV only)."""
    lib = load_library()
    B, H, N, d = o.shape
    _check_tensor(o, "o", (B, H, N, d))
    _check_tensor(dout, "dout", (B, H, N, d), device=o.device)
    _check_tensor(lse, "lse", (B, H, N), dtype=torch.float32, device=o.device)
    st = lib.fa2_bwd_preprocess(o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                *_ws(workspace, o.device, B, H, N, d), B, H, N, d,
                                _stream_ptr(o.device))
    _check(st, "fa2_bwd_preprocess")
    return workspace


def bwd_dkdv(q, k, v, dout, workspace, causal=False, scale=None, dk=None, dv=None):
    """dK, dV from q, k, v, dout and a workspace filled by bwd_dq (or bwd_preprocess)."""
    lib = load_library()
    B, H, N, d = q.shape
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check_tensor(t, nm, (B, H, N, d), device=q.device)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor(dk, "dk", (B, H, N, d), device=q.device)
    _check_tensor(dv, "dv", (B, H, N, d), device=q.device)
    s = default_scale(d) if scale is None else float(scale)
    st = lib.fa2_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                          *_ws(workspace, q.device, B, H, N, d), dk.data_ptr(), dv.data_ptr(),
                          B, H, N, d, int(bool(causal)), s, _stream_ptr(q.device))
    _check(st, "fa2_bwd_dkdv")
    return dk, dv


def bwd_dq(q, k, v, o, dout, lse, workspace, causal=False, scale=None, dq=None):
    """dQ from q, k, v, o, dout and lse; also fills `workspace` (D, LSE * log2(e)) for
    bwd_dkdv."""
    lib = load_library()
    B, H, N, d = q.shape
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check_tensor(t, nm, (B, H, N, d), device=q.device)
    _check_tensor(lse, "lse", (B, H, N), dtype=torch.float32, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    _check_tensor(dq, "dq", (B, H, N, d), device=q.device)
    s = default_scale(d) if scale is None else float(scale)
    st = lib.fa2_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        dout.data_ptr(), lse.data_ptr(), *_ws(workspace, q.device, B, H, N, d),
                        dq.data_ptr(), B, H, N, d, int(bool(causal)), s, _stream_ptr(q.device))
    _check(st, "fa2_bwd_dq")
    return dq
