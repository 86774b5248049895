"""Dynamic top-k sparse attention on MI355X (gfx950).

Thin Python binding of libsparse_attn.so (include/sparse_attn.h): every
function here only checks and marshals torch tensors (device pointers and the
current HIP stream) and calls the C entry point of the same name; all
arithmetic runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing or the tensors are not on a GPU the call raises.

The method (page "mhpq.cn/news/1098205", §1.3 and §2.2): a low-dimensional
scorer q_low = Q·Pq, k_low = K·Pk scores every pair as
d_proj^-1/2 · q_low·k_low, each query keeps its k best keys, and
softmax(q·K_selᵀ/√D)·V_sel runs over those keys only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsparse_attn.so")

SA_F32, SA_BF16, SA_F16 = 0, 1, 2
SA_OK = 0
SA_K_MAX = 2048
STATUS_NAMES = {
    0: "SA_OK", -1: "SA_ERR_NULL", -2: "SA_ERR_SHAPE", -3: "SA_ERR_UNSUPPORTED",
    -4: "SA_ERR_ALIGN", -5: "SA_ERR_WORKSPACE", -6: "SA_ERR_HIP", -7: "SA_ERR_DEVICE_INDEX",
}

# every symbol include/sparse_attn.h declares
EXPORTS = (
    "sparse_attn_workspace_size", "sparse_attn_workspace_size_for_chunk",
    "sparse_attn_scores_topk", "sparse_attn_gather", "sparse_attn_fwd",
    "sparse_attn_band_indices", "sparse_attn_scores_dump", "sparse_attn_check_status",
    "sparse_attn_workspace_stats", "sparse_attn_profile_enable", "sparse_attn_profile_read",
    "sparse_attn_set_filter_dtype", "sparse_attn_get_filter_dtype", "sparse_attn_status_string",
)


class sa_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32)]


class sa_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("ms", ctypes.c_float)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsparse_attn.so (built by dynamic_top_sparse_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m dynamic_top_sparse_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "sparse_attn_workspace_size": (sz, [sa_dims, i32, i32, i32, i32, i32]),
        "sparse_attn_workspace_size_for_chunk": (sz, [sa_dims, i32, i32, i32, i32, i32, i32]),
        "sparse_attn_scores_topk": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32, i32, f32,
                                                   i32, vp, vp, sz, vp]),
        "sparse_attn_gather": (ctypes.c_int, [vp, vp, vp, vp, i32, sa_dims, f32, i32, vp, vp]),
        "sparse_attn_fwd": (ctypes.c_int, [vp, vp, vp, vp, vp, sa_dims, i32, i32, i32, f32, f32,
                                           i32, vp, vp, vp, sz, vp]),
        "sparse_attn_band_indices": (ctypes.c_int, [sa_dims, i32, i32, vp, i32, vp]),
        "sparse_attn_scores_dump": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32, f32, i32,
                                                   i32, i32, vp, vp, sz, vp]),
        "sparse_attn_check_status": (ctypes.c_int, [vp]),
        "sparse_attn_workspace_stats": (ctypes.c_int, [vp, sz, ctypes.POINTER(ctypes.c_int64),
                                                       i32, vp]),
        "sparse_attn_profile_enable": (ctypes.c_int, [i32]),
        "sparse_attn_profile_read": (ctypes.c_int, [ctypes.POINTER(sa_kernel_time), i32]),
        "sparse_attn_set_filter_dtype": (ctypes.c_int, [i32]),
        "sparse_attn_get_filter_dtype": (ctypes.c_int, []),
        "sparse_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().sparse_attn_status_string(status).decode()
    except Exception:  # the library is not loadable: report the code only
        return STATUS_NAMES.get(status, "unknown status")


# ------------------------------------------------------------- helpers ---

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dims(Q: torch.Tensor) -> sa_dims:
    if Q.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, D]")
    B, H, N, D = Q.shape
    return sa_dims(B, H, N, D)


def _check(status: int, where: str) -> None:
    if status != SA_OK:
        raise SparseAttnError(status, where)


def default_score_scale(d_proj: int) -> float:
    """d_proj^-1/2, the scorer's scale (page "mhpq.cn/news/1098205", §2.2)."""
    return float(d_proj) ** -0.5


def default_softmax_scale(D: int) -> float:
    """D^-1/2, the attention scale (same page, §1.2 and §3.2)."""
    return float(D) ** -0.5


# -------------------------------------------------------- entry points ---

def sparse_attn_workspace_size(B: int, H: int, N: int, D: int, d_proj: int, k: int,
                               causal: bool, dtype: torch.dtype, with_idx: bool = False,
                               heads_per_chunk: Optional[int] = None) -> int:
    code = SA_F32 if dtype == torch.float32 else SA_BF16
    lib = load_library()
    d = sa_dims(B, H, N, D)
    if heads_per_chunk is None:
        return int(lib.sparse_attn_workspace_size(d, d_proj, k, int(causal), code, int(with_idx)))
    return int(lib.sparse_attn_workspace_size_for_chunk(d, d_proj, k, int(causal), code,
                                                        int(with_idx), heads_per_chunk))


def allocate_workspace(Q: torch.Tensor, d_proj: int, k: int, causal: bool,
                       with_idx: bool = False, heads_per_chunk: Optional[int] = None) -> torch.Tensor:
    B, H, N, D = Q.shape
    n = sparse_attn_workspace_size(B, H, N, D, d_proj, k, causal, Q.dtype, with_idx,
                                   heads_per_chunk)
    if n == 0:
        raise SparseAttnError(-3, "sparse_attn_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=Q.device)


def sparse_attn_scores_topk(Q, K, Pq, Pk, k: int, causal: bool = False,
                            score_scale: Optional[float] = None,
                            idx: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """idx [B,H,N,k] int32: each query's k best keys by the scorer, ascending
    key order, -1 padded (see include/sparse_attn.h)."""
    B, H, N, D = Q.shape
    d_proj = Pq.shape[1]
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    if idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=Q.device)
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, k, causal)
    st = load_library().sparse_attn_scores_topk(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj, k,
        int(causal), scale, _dtype_code(Q), _dev(idx, "idx"), _dev(workspace, "workspace"),
        workspace.numel(), _stream(Q))
    _check(st, "sparse_attn_scores_topk")
    return idx


def sparse_attn_gather(Q, K, V, idx, softmax_scale: Optional[float] = None,
                       O: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O [B,H,N,D]: softmax attention of each query over its idx row."""
    B, H, N, D = Q.shape
    k = idx.shape[-1]
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    if O is None:
        O = torch.empty_like(Q)
    st = load_library().sparse_attn_gather(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(idx, "idx"), k, _dims(Q), scale,
        _dtype_code(Q), _dev(O, "O"), _stream(Q))
    _check(st, "sparse_attn_gather")
    return O


def sparse_attn_fwd(Q, K, V, Pq, Pk, k: int, causal: bool = False,
                    score_scale: Optional[float] = None, softmax_scale: Optional[float] = None,
                    O: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, return_idx: bool = False):
    """The fused forward; returns O (and idx when return_idx)."""
    B, H, N, D = Q.shape
    d_proj = Pq.shape[1]
    sscale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    ascale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    if O is None:
        O = torch.empty_like(Q)
    if return_idx and idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=Q.device)
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, k, causal, with_idx=idx is None)
    st = load_library().sparse_attn_fwd(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q),
        d_proj, k, int(causal), sscale, ascale, _dtype_code(Q), _dev(O, "O"),
        None if idx is None else _dev(idx, "idx"), _dev(workspace, "workspace"),
        workspace.numel(), _stream(Q))
    _check(st, "sparse_attn_fwd")
    return (O, idx) if return_idx else O


def sparse_attn_band_indices(B: int, H: int, N: int, w_left: int, w_right: int,
                             k: Optional[int] = None, device="cuda",
                             idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """idx [B,H,N,k]: keys max(0,i-w_left)..min(N-1,i+w_right), then -1."""
    if k is None:
        k = w_left + w_right + 1
    if idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=device)
    st = load_library().sparse_attn_band_indices(sa_dims(B, H, N, 0), w_left, w_right,
                                                 _dev(idx, "idx"), k, _stream(idx))
    _check(st, "sparse_attn_band_indices")
    return idx


def sparse_attn_scores_dump(Q, K, Pq, Pk, row_begin: int, row_count: int,
                            causal: bool = False, score_scale: Optional[float] = None,
                            S: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S [B,H,row_count,N] fp32: the exact scores the selection uses."""
    B, H, N, D = Q.shape
    d_proj = Pq.shape[1]
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    if S is None:
        S = torch.empty((B, H, row_count, N), dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, 1, causal)
    st = load_library().sparse_attn_scores_dump(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj,
        int(causal), scale, _dtype_code(Q), row_begin, row_count, _dev(S, "S"),
        _dev(workspace, "workspace"), workspace.numel(), _stream(Q))
    _check(st, "sparse_attn_scores_dump")
    return S


def sparse_attn_check_status(stream: Optional[int] = None) -> int:
    """Synchronizes and returns SA_OK or SA_ERR_DEVICE_INDEX (clearing it)."""
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    return int(load_library().sparse_attn_check_status(s))


def sparse_attn_workspace_stats(workspace: torch.Tensor) -> dict:
    out = (ctypes.c_int64 * 6)()
    n = load_library().sparse_attn_workspace_stats(
        _dev(workspace, "workspace"), workspace.numel(), out, 6, _stream(workspace))
    if n < 0:
        raise SparseAttnError(n, "sparse_attn_workspace_stats")
    keys = ("fallback_queries", "overflow_queries", "candidates", "rescored", "queries",
            "retried")
    return {kk: int(out[i]) for i, kk in enumerate(keys[:n])}


def sparse_attn_set_filter_dtype(dtype: torch.dtype) -> None:
    """16-bit operand type of the MFMA filter: torch.float16 (default) or
    torch.bfloat16.  Indices do not depend on it (see include/sparse_attn.h)."""
    code = {torch.float16: SA_F16, torch.bfloat16: SA_BF16}[dtype]
    _check(load_library().sparse_attn_set_filter_dtype(code), "sparse_attn_set_filter_dtype")


def sparse_attn_get_filter_dtype() -> torch.dtype:
    return torch.float16 if load_library().sparse_attn_get_filter_dtype() == SA_F16 else torch.bfloat16


def sparse_attn_profile_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (for benchmarks)."""
    _check(load_library().sparse_attn_profile_enable(int(on)), "sparse_attn_profile_enable")


def sparse_attn_profile_read(max_records: int = 65536) -> list:
    """[(kernel name, ms)] of the launches timed since the last read."""
    buf = (sa_kernel_time * max_records)()
    n = load_library().sparse_attn_profile_read(buf, max_records)
    if n < 0:
        raise SparseAttnError(n, "sparse_attn_profile_read")
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]


__all__ = [
    "sa_dims", "SparseAttnError", "load_library", "status_string", "LIB_PATH", "EXPORTS",
    "sparse_attn_workspace_size", "allocate_workspace", "sparse_attn_scores_topk",
    "sparse_attn_gather", "sparse_attn_fwd", "sparse_attn_band_indices",
    "sparse_attn_scores_dump", "sparse_attn_check_status", "sparse_attn_workspace_stats",
    "default_score_scale", "default_softmax_scale", "sparse_attn_profile_enable",
    "sparse_attn_profile_read", "sparse_attn_set_filter_dtype", "sparse_attn_get_filter_dtype",
]
