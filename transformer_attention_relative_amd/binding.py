"""Thin ctypes binding over ``librelattn.so`` (declared in include/relattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

from .build import LIB_PATH

# relattn_params layout this binding marshals (RELATTN_ABI_VERSION in the header)
ABI_VERSION = 2

KINDS = {"t5": 0, "shaw": 1, "deberta": 2, "alibi": 3, "txl": 4}
DTYPES = {"fp32": 0, "bf16": 1}
STATUS = {0: "RELATTN_OK", 1: "RELATTN_ERR_INVALID", 2: "RELATTN_ERR_UNSUPPORTED",
          3: "RELATTN_ERR_WORKSPACE", 4: "RELATTN_ERR_HIP"}


class RelattnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class relattn_params(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Lq", ctypes.c_int32),
        ("Lk", ctypes.c_int32), ("d", ctypes.c_int32),
        ("table", ctypes.c_void_p), ("table2", ctypes.c_void_p),
        ("num_buckets", ctypes.c_int32), ("max_distance", ctypes.c_int32),
        ("bidirectional", ctypes.c_int32), ("clip_k", ctypes.c_int32),
        ("q_pos_offset", ctypes.c_int32), ("k_pos_offset", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("kv_valid_len", ctypes.c_void_p), ("scale", ctypes.c_float),
        ("lse", ctypes.c_void_p),
    ]


EXPORTS = ("relattn_fwd", "relattn_fwd_noalloc", "relattn_workspace_bytes", "relattn_rel_index",
           "relattn_t5_thresholds", "relattn_status_str", "relattn_last_error",
           "relattn_abi_version")
# bytes of the fixed device scratch behind relattn_fwd_noalloc
NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None
_lock = threading.Lock()


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) the built library; raise if it is not there."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or os.environ.get("RELATTN_LIB", LIB_PATH)
        if not os.path.exists(p):
            raise RuntimeError(f"{p} not found: build it with "
                               "`python -m transformer_attention_relative_amd.build`")
        lib = ctypes.CDLL(p)
        P = ctypes.POINTER(relattn_params)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.relattn_fwd.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        lib.relattn_fwd.restype = i32
        lib.relattn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp]
        lib.relattn_fwd_noalloc.restype = i32
        lib.relattn_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
        lib.relattn_workspace_bytes.restype = i32
        lib.relattn_rel_index.argtypes = [P, vp, vp, i64, i32, vp, vp]
        lib.relattn_rel_index.restype = i32
        lib.relattn_t5_thresholds.argtypes = [i32, i32, i32, ctypes.POINTER(i32), i32,
                                              ctypes.POINTER(i32)]
        lib.relattn_t5_thresholds.restype = i32
        lib.relattn_status_str.argtypes = [i32]
        lib.relattn_status_str.restype = ctypes.c_char_p
        lib.relattn_last_error.argtypes = []
        lib.relattn_last_error.restype = ctypes.c_char_p
        lib.relattn_abi_version.argtypes = []
        lib.relattn_abi_version.restype = i32
        # a library built for another parameter layout would read every
        # field after the first difference from the wrong offset (pointers
        # included): refuse it before any call
        got = lib.relattn_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(f"{p}: ABI version {got}, this binding marshals version "
                               f"{ABI_VERSION}; rebuild the library")
        if path is None:
            _lib = lib
        return lib


def _check(lib, status: int):
    if status != 0:
        raise RelattnError(status, lib.relattn_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_params(kind: str, dtype: str, B: int, H: int, Lq: int, Lk: int, d: int, *,
                table=None, table2=None, num_buckets: int = 32, max_distance: int = 128,
                bidirectional: bool = True, clip_k: int = 0, q_pos_offset: int = 0,
                k_pos_offset: int = 0, causal: bool = False, kv_valid_len=None,
                scale: float = 0.0, lse=None) -> relattn_params:
    return relattn_params(
        KINDS[kind], DTYPES[dtype], B, H, Lq, Lk, d, _ptr(table), _ptr(table2),
        num_buckets, max_distance, int(bool(bidirectional)), clip_k, q_pos_offset,
        k_pos_offset, int(bool(causal)), _ptr(kv_valid_len), float(scale), _ptr(lse))


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def relattn_workspace_bytes(params: relattn_params) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib, lib.relattn_workspace_bytes(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def _table_specs(kind: str, dtype, H: int, d: int, clip_k: int, num_buckets: int):
    """(dtype, shape) of table and table2 for a kind, as include/relattn.h
    states them (None: the table must be absent)."""
    import torch
    if kind == "t5":
        return (torch.float32, (num_buckets, H)), None
    if kind == "alibi":
        return (torch.float32, (H,)), None
    if kind == "shaw":
        n = 2 * clip_k + 1
        return (dtype, (n, d)), (dtype, (n, d))
    if kind == "deberta":
        n = 2 * clip_k
        return (dtype, (n, H, d)), (dtype, (n, H, d))
    if kind == "txl":
        return (dtype, (clip_k, H, d)), (dtype, (2, H, d))
    raise ValueError(f"unknown kind {kind!r}")


def _check_tensor(name, t, dtype=None, shape=None):
    """dtype and shape first, then contiguity; the device is checked last
    (by _check_device), so the layout errors show on any machine."""
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != device):
            raise ValueError(f"{name} must be a GPU tensor on {device} (got {t.device})")


def relattn_fwd(q, k, v, kind: str, table=None, table2=None, *, num_buckets: int = 32,
                max_distance: int = 128, bidirectional: bool = True, clip_k: int = 0,
                q_pos_offset: int = 0, k_pos_offset: int = 0, causal: bool = False,
                kv_valid_len=None, scale: float = 0.0, out=None, workspace=None, lse=None):
    """Fused forward on the current HIP stream; returns ``out``.

    q [B, H, Lq, d], k/v [B, H, Lk, d] (float32 or bfloat16, contiguous, on
    the GPU).  Tables: T5 float32 [num_buckets, H]; Shaw a_K / a_V
    [2k+1, d]; DeBERTa Kr / Qr [2k, H, d] (input dtype); ALiBi float32
    slopes [H]; Transformer-XL encodings E [clip_k, H, d] and (u, v)
    [2, H, d] (input dtype).  Query row i sits at
    absolute position ``q_pos_offset + i``, key row j at ``k_pos_offset + j``.
    ``kv_valid_len``:
    int32 [B] on the GPU or None.  ``out`` ([B, H, Lq, d], q's dtype) and
    ``workspace`` (any dtype, at least ``relattn_workspace_bytes`` bytes) are
    allocated with torch when not given.  ``lse``: a float32 [B, H, Lq] GPU
    tensor that receives each row's log-sum-exp of the logits (natural log),
    or None.  Every tensor's dtype, shape, layout and device is checked here
    before the library is called.
    """
    import torch
    lib, p, out = _checked_call(q, k, v, kind, table, table2, num_buckets, max_distance,
                                bidirectional, clip_k, q_pos_offset, k_pos_offset, causal,
                                kv_valid_len, scale, out, workspace, lse)
    nbytes = relattn_workspace_bytes(p)
    if nbytes and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if nbytes else None
    ws_len = workspace.numel() * workspace.element_size() if (nbytes and workspace is not None) else 0
    _check(lib, lib.relattn_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), ws_ptr, ws_len, _stream_handle(q.device)))
    return out


def relattn_fwd_noalloc(q, k, v, kind: str, table=None, table2=None, *, out, num_buckets: int = 32,
                        max_distance: int = 128, bidirectional: bool = True, clip_k: int = 0,
                        q_pos_offset: int = 0, k_pos_offset: int = 0, causal: bool = False,
                        kv_valid_len=None, scale: float = 0.0, lse=None):
    """relattn_fwd without a workspace: the library's fixed device scratch
    (one per GPU) holds it, and nothing is allocated; ``out`` must be given.
    Calls that overlap in time on one GPU share that scratch and must be
    ordered by the caller (include/relattn.h)."""
    if out is None:
        raise ValueError("relattn_fwd_noalloc writes into a given `out`")
    lib, p, out = _checked_call(q, k, v, kind, table, table2, num_buckets, max_distance,
                                bidirectional, clip_k, q_pos_offset, k_pos_offset, causal,
                                kv_valid_len, scale, out, None, lse)
    _check(lib, lib.relattn_fwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), out.data_ptr(), _stream_handle(q.device)))
    return out


def _checked_call(q, k, v, kind, table, table2, num_buckets, max_distance, bidirectional,
                  clip_k, q_pos_offset, k_pos_offset, causal, kv_valid_len, scale, out,
                  workspace, lse):
    """Check every tensor, load the library; return (lib, params, out)."""
    import torch
    if kind not in KINDS:
        raise ValueError(f"unknown kind {kind!r}")
    if q.dtype == torch.float32:
        dtype = "fp32"
    elif q.dtype == torch.bfloat16:
        dtype = "bf16"
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k and v must be 4-D [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    _check_tensor("q", q)
    _check_tensor("k", k, q.dtype, (B, H, Lk, d))
    _check_tensor("v", v, q.dtype, (B, H, Lk, d))
    spec1, spec2 = _table_specs(kind, q.dtype, H, d, clip_k, num_buckets)
    if table is None:
        raise ValueError(f"{kind} needs table {spec1[1]}")
    _check_tensor("table", table, *spec1)
    if spec2 is None:
        if table2 is not None:
            raise ValueError(f"{kind} takes no table2")
    else:
        if table2 is None:
            raise ValueError(f"{kind} needs table2 {spec2[1]}")
        _check_tensor("table2", table2, *spec2)
    if kv_valid_len is not None:
        _check_tensor("kv_valid_len", kv_valid_len, torch.int32)
        if kv_valid_len.numel() < B:
            raise ValueError(f"kv_valid_len needs {B} entries (got {kv_valid_len.numel()})")
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, (B, H, Lq))
    if out is not None:
        _check_tensor("out", out, q.dtype, (B, H, Lq, d))
    if workspace is not None:
        _check_tensor("workspace", workspace)
    _check_device(q.device, q=q, k=k, v=v, table=table, table2=table2,
                  kv_valid_len=kv_valid_len, lse=lse, out=out, workspace=workspace)
    lib = load_library()
    p = make_params(kind, dtype, B, H, Lq, Lk, d, table=table, table2=table2,
                    num_buckets=num_buckets, max_distance=max_distance,
                    bidirectional=bidirectional, clip_k=clip_k, q_pos_offset=q_pos_offset,
                    k_pos_offset=k_pos_offset, causal=causal, kv_valid_len=kv_valid_len,
                    scale=scale, lse=lse)
    if out is None:
        out = torch.empty_like(q)
    return lib, p, out


def relattn_rel_index(kind: str, q_pos, k_pos, which: int = 0, *, num_buckets: int = 32,
                      max_distance: int = 128, bidirectional: bool = True, clip_k: int = 0,
                      out=None):
    """Index of each (q_pos[e], k_pos[e]) pair (int32 GPU tensors) on the GPU."""
    import torch
    if kind not in KINDS:
        raise ValueError(f"unknown kind {kind!r}")
    _check_tensor("q_pos", q_pos, torch.int32)
    _check_tensor("k_pos", k_pos, torch.int32, tuple(q_pos.shape))
    if out is not None:
        _check_tensor("out", out, torch.int32, tuple(q_pos.shape))
    _check_device(q_pos.device, q_pos=q_pos, k_pos=k_pos, out=out)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q_pos)
    p = make_params(kind, "fp32", 1, 1, 1, 1, 32, num_buckets=num_buckets,
                    max_distance=max_distance, bidirectional=bidirectional, clip_k=clip_k)
    _check(lib, lib.relattn_rel_index(ctypes.byref(p), q_pos.data_ptr(), k_pos.data_ptr(),
                                      q_pos.numel(), which, out.data_ptr(),
                                      _stream_handle(q_pos.device)))
    return out


def relattn_t5_thresholds(num_buckets: int = 32, max_distance: int = 128,
                          bidirectional: bool = True) -> list:
    """Host-computed T5 slot thresholds (see include/relattn.h)."""
    lib = load_library()
    buf = (ctypes.c_int32 * 256)()
    cnt = ctypes.c_int32(0)
    _check(lib, lib.relattn_t5_thresholds(num_buckets, max_distance, int(bool(bidirectional)),
                                          buf, 256, ctypes.byref(cnt)))
    return list(buf[: cnt.value])
