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
    "sparse_attn_workspace_stats", "sparse_attn_profile_create", "sparse_attn_profile_destroy",
    "sparse_attn_profile_read", "sparse_attn_status_string",
    "sparse_attn_scores_topk_smoothed", "sparse_attn_dilated_indices",
    "sparse_attn_band_indices_per_batch", "sparse_attn_decode_workspace_size",
    "sparse_attn_decode_append_keys", "sparse_attn_decode", "sparse_attn_block_workspace_size",
    "sparse_attn_block_topk", "sparse_attn_block_scores_dump", "sparse_attn_bwd_workspace_size",
    "sparse_attn_bwd", "sparse_attn_decode_noalloc_max_bytes", "sparse_attn_decode_noalloc",
    "sparse_attn_gather_workspace_size", "sparse_attn_gather_ws",
)


class sa_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32)]


class sa_options(ctypes.Structure):
    _fields_ = [("filter_dtype", ctypes.c_int32), ("profile", ctypes.c_void_p),
                ("bwd_parts", ctypes.c_int32)]


BWD_PARTS = {"auto": 0, "whole": 1, "split": 2}


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
    op = ctypes.POINTER(sa_options)
    sig = {
        "sparse_attn_workspace_size": (sz, [sa_dims, i32, i32, i32, i32, i32]),
        "sparse_attn_workspace_size_for_chunk": (sz, [sa_dims, i32, i32, i32, i32, i32, i32]),
        "sparse_attn_scores_topk": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32, i32, f32,
                                                   i32, vp, vp, sz, op, vp]),
        "sparse_attn_gather": (ctypes.c_int, [vp, vp, vp, vp, i32, sa_dims, f32, i32, vp, op,
                                              vp]),
        "sparse_attn_gather_workspace_size": (sz, [sa_dims, i32, i32]),
        "sparse_attn_gather_ws": (ctypes.c_int, [vp, vp, vp, vp, i32, sa_dims, f32, i32, vp, vp,
                                                 sz, op, vp]),
        "sparse_attn_fwd": (ctypes.c_int, [vp, vp, vp, vp, vp, sa_dims, i32, i32, i32, f32, f32,
                                           i32, vp, vp, vp, sz, op, vp]),
        "sparse_attn_band_indices": (ctypes.c_int, [sa_dims, i32, i32, vp, i32, op, vp]),
        "sparse_attn_scores_dump": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32, f32, i32,
                                                   i32, i32, vp, vp, sz, op, vp]),
        "sparse_attn_check_status": (ctypes.c_int, [vp]),
        "sparse_attn_workspace_stats": (ctypes.c_int, [vp, sz, ctypes.POINTER(ctypes.c_int64),
                                                       i32, vp]),
        "sparse_attn_profile_create": (vp, []),
        "sparse_attn_profile_destroy": (None, [vp]),
        "sparse_attn_profile_read": (ctypes.c_int, [vp, ctypes.POINTER(sa_kernel_time), i32]),
        "sparse_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "sparse_attn_scores_topk_smoothed": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32,
                                                            i32, f32, f32, i32, vp, vp, sz, op,
                                                            vp]),
        "sparse_attn_dilated_indices": (ctypes.c_int, [sa_dims, i32, i32, vp, i32, op, vp]),
        "sparse_attn_band_indices_per_batch": (ctypes.c_int, [sa_dims, vp, vp, i32, op, vp]),
        "sparse_attn_decode_workspace_size": (sz, [sa_dims, i32, i32]),
        "sparse_attn_decode_append_keys": (ctypes.c_int, [vp, vp, sa_dims, i32, i32, vp, i32, i32,
                                                          op, vp]),
        "sparse_attn_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, sa_dims, i32, i32, i32, f32,
                                              f32, i32, vp, vp, vp, vp, sz, op, vp]),
        "sparse_attn_block_workspace_size": (sz, [sa_dims, i32, i32, i32]),
        "sparse_attn_bwd_workspace_size": (sz, [sa_dims, i32, i32, i32, op]),
        "sparse_attn_decode_noalloc_max_bytes": (sz, []),
        "sparse_attn_decode_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, sa_dims, i32, i32, i32,
                                                      f32, f32, i32, vp, vp, vp, vp]),
        "sparse_attn_bwd": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, sa_dims, i32, i32, f32, f32,
                                           i32, vp, vp, vp, vp, vp, vp, sz, op, vp]),
        "sparse_attn_block_topk": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32, i32, i32,
                                                  f32, i32, vp, vp, sz, op, vp]),
        "sparse_attn_block_scores_dump": (ctypes.c_int, [vp, vp, vp, vp, sa_dims, i32, i32, f32,
                                                         i32, i32, i32, vp, vp, sz, op, vp]),
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


class Profile:
    """A caller-owned per-kernel timing record (sa_profile): pass it as
    ``profile=`` to a call; read() returns [(kernel name, ms)] of the launches
    recorded since the last read."""

    def __init__(self):
        self._lib = load_library()
        self.handle = self._lib.sparse_attn_profile_create()
        if not self.handle:
            raise RuntimeError("sparse_attn_profile_create failed")

    def read(self, max_records: int = 65536) -> list:
        buf = (sa_kernel_time * max_records)()
        n = self._lib.sparse_attn_profile_read(self.handle, buf, max_records)
        if n < 0:
            raise SparseAttnError(n, "sparse_attn_profile_read")
        return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]

    def close(self) -> None:
        if self.handle:
            self._lib.sparse_attn_profile_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------- helpers ---

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _filter_code(dtype) -> int:
    if dtype is None or dtype == torch.float16:
        return SA_F16
    if dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError(f"filter dtype must be torch.float16 or torch.bfloat16, not {dtype}")


def _options(filter_dtype=None, profile: Optional[Profile] = None, bwd_parts: str = "auto"):
    if bwd_parts not in BWD_PARTS:
        raise ValueError(f"bwd_parts must be one of {sorted(BWD_PARTS)}")
    return ctypes.byref(sa_options(_filter_code(filter_dtype),
                                   profile.handle if profile is not None else None,
                                   BWD_PARTS[bwd_parts]))


def _tensor(t, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    return t


def _like(t, ref: torch.Tensor, name: str, ref_name: str) -> None:
    """t must have ref's shape, dtype and device."""
    _tensor(t, name)
    if tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, {ref_name} {tuple(ref.shape)}")
    if t.dtype != ref.dtype:
        raise ValueError(f"{name} is {t.dtype} but {ref_name} is {ref.dtype}: one dtype for all")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _check_qkv(Q, K, V=None, O=None) -> None:
    _tensor(Q, "Q")
    if Q.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, D]")
    _dtype_code(Q)
    _like(K, Q, "K", "Q")
    if V is not None:
        _like(V, Q, "V", "Q")
    if O is not None:
        _like(O, Q, "O", "Q")


def _check_proj(Pq, Pk, Q) -> int:
    _tensor(Pq, "Pq")
    _tensor(Pk, "Pk")
    D = Q.shape[3]
    if Pq.dim() != 2 or Pq.shape[0] != D:
        raise ValueError(f"Pq must be [D, d_proj] = [{D}, d_proj], got {tuple(Pq.shape)}")
    _like(Pk, Pq, "Pk", "Pq")
    if Pq.dtype != Q.dtype or Pq.device != Q.device:
        raise ValueError("Pq and Pk must have Q's dtype and device")
    return int(Pq.shape[1])


def _check_idx(idx, Q, k: int, name: str = "idx") -> None:
    _tensor(idx, name)
    B, H, N, _ = Q.shape
    if idx.dtype != torch.int32:
        raise ValueError(f"{name} must be int32, got {idx.dtype}")
    if tuple(idx.shape) != (B, H, N, k):
        raise ValueError(f"{name} must be [B, H, N, k] = {(B, H, N, k)}, got {tuple(idx.shape)}")
    if idx.device != Q.device:
        raise ValueError(f"{name} is on {idx.device}, Q on {Q.device}")


def _dev(t: torch.Tensor, name: str) -> int:
    _tensor(t, name)
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


def _check_workspace(ws, Q) -> None:
    _tensor(ws, "workspace")
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if ws.device != Q.device:
        raise ValueError(f"workspace is on {ws.device}, Q on {Q.device}")


def sparse_attn_scores_topk(Q, K, Pq, Pk, k: int, causal: bool = False,
                            score_scale: Optional[float] = None,
                            idx: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None,
                            filter_dtype: Optional[torch.dtype] = None,
                            profile: Optional[Profile] = None) -> torch.Tensor:
    """idx [B,H,N,k] int32: each query's k best keys by the scorer, ascending
    key order, -1 padded (see include/sparse_attn.h)."""
    _check_qkv(Q, K)
    d_proj = _check_proj(Pq, Pk, Q)
    B, H, N, D = Q.shape
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    if idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=Q.device)
    _check_idx(idx, Q, k)
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, k, causal)
    _check_workspace(workspace, Q)
    st = load_library().sparse_attn_scores_topk(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj, k,
        int(causal), scale, _dtype_code(Q), _dev(idx, "idx"), _dev(workspace, "workspace"),
        workspace.numel(), _options(filter_dtype, profile), _stream(Q))
    _check(st, "sparse_attn_scores_topk")
    return idx


def sparse_attn_gather(Q, K, V, idx, softmax_scale: Optional[float] = None,
                       O: Optional[torch.Tensor] = None,
                       profile: Optional[Profile] = None, by_range: bool = True,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O [B,H,N,D]: softmax attention of each query over its idx row.  With
    by_range (the default) the call is sparse_attn_gather_ws, which takes
    rows of ascending keys by key range when N is large (a workspace of
    sparse_attn_gather_workspace_size bytes, allocated here unless given);
    otherwise sparse_attn_gather, one pass per row."""
    _check_qkv(Q, K, V, O)
    B, H, N, D = Q.shape
    _tensor(idx, "idx")
    if idx.dim() != 4:
        raise ValueError("idx must be [B, H, N, k]")
    k = idx.shape[-1]
    _check_idx(idx, Q, k)
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    if O is None:
        O = torch.empty_like(Q)
    lib = load_library()
    n_ws = int(lib.sparse_attn_gather_workspace_size(_dims(Q), k, _dtype_code(Q))) \
        if by_range else 0
    if n_ws > 0:
        if workspace is None:
            workspace = torch.empty(n_ws, dtype=torch.uint8, device=Q.device)
        _tensor(workspace, "workspace")
        if workspace.dtype != torch.uint8 or workspace.device != Q.device:
            raise ValueError("workspace must be a uint8 tensor on Q's device")
        st = lib.sparse_attn_gather_ws(
            _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(idx, "idx"), k, _dims(Q), scale,
            _dtype_code(Q), _dev(O, "O"), _dev(workspace, "workspace"), workspace.numel(),
            _options(None, profile), _stream(Q))
        _check(st, "sparse_attn_gather_ws")
        return O
    st = lib.sparse_attn_gather(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(idx, "idx"), k, _dims(Q), scale,
        _dtype_code(Q), _dev(O, "O"), _options(None, profile), _stream(Q))
    _check(st, "sparse_attn_gather")
    return O


def sparse_attn_fwd(Q, K, V, Pq, Pk, k: int, causal: bool = False,
                    score_scale: Optional[float] = None, softmax_scale: Optional[float] = None,
                    O: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, return_idx: bool = False,
                    filter_dtype: Optional[torch.dtype] = None,
                    profile: Optional[Profile] = None):
    """The fused forward; returns O (and idx when return_idx)."""
    _check_qkv(Q, K, V, O)
    d_proj = _check_proj(Pq, Pk, Q)
    B, H, N, D = Q.shape
    sscale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    ascale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    if O is None:
        O = torch.empty_like(Q)
    if return_idx and idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=Q.device)
    if idx is not None:
        _check_idx(idx, Q, k)
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, k, causal, with_idx=idx is None)
    _check_workspace(workspace, Q)
    st = load_library().sparse_attn_fwd(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q),
        d_proj, k, int(causal), sscale, ascale, _dtype_code(Q), _dev(O, "O"),
        None if idx is None else _dev(idx, "idx"), _dev(workspace, "workspace"),
        workspace.numel(), _options(filter_dtype, profile), _stream(Q))
    _check(st, "sparse_attn_fwd")
    return (O, idx) if return_idx else O


def sparse_attn_band_indices(B: int, H: int, N: int, w_left: int, w_right: int,
                             k: Optional[int] = None, device="cuda",
                             idx: Optional[torch.Tensor] = None,
                             profile: Optional[Profile] = None) -> torch.Tensor:
    """idx [B,H,N,k]: keys max(0,i-w_left)..min(N-1,i+w_right), then -1."""
    if k is None:
        k = w_left + w_right + 1
    if idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=device)
    _tensor(idx, "idx")
    if idx.dtype != torch.int32 or tuple(idx.shape) != (B, H, N, k):
        raise ValueError(f"idx must be int32 [B, H, N, k] = {(B, H, N, k)}")
    st = load_library().sparse_attn_band_indices(sa_dims(B, H, N, 0), w_left, w_right,
                                                 _dev(idx, "idx"), k, _options(None, profile),
                                                 _stream(idx))
    _check(st, "sparse_attn_band_indices")
    return idx


def sparse_attn_scores_topk_smoothed(Q, K, Pq, Pk, k: int, gap: float, causal: bool = False,
                                     score_scale: Optional[float] = None,
                                     idx: Optional[torch.Tensor] = None,
                                     workspace: Optional[torch.Tensor] = None,
                                     filter_dtype: Optional[torch.dtype] = None,
                                     profile: Optional[Profile] = None) -> torch.Tensor:
    """idx [B,H,N,k+1] int32: the top-k, plus the (k+1)-th key where the
    score gap to the k-th is below `gap` (boundary smoothing)."""
    _check_qkv(Q, K)
    d_proj = _check_proj(Pq, Pk, Q)
    B, H, N, D = Q.shape
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    if idx is None:
        idx = torch.empty((B, H, N, k + 1), dtype=torch.int32, device=Q.device)
    _check_idx(idx, Q, k + 1)
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, k + 1, causal)
    _check_workspace(workspace, Q)
    st = load_library().sparse_attn_scores_topk_smoothed(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj, k,
        int(causal), scale, float(gap), _dtype_code(Q), _dev(idx, "idx"),
        _dev(workspace, "workspace"), workspace.numel(), _options(filter_dtype, profile),
        _stream(Q))
    _check(st, "sparse_attn_scores_topk_smoothed")
    return idx


def sparse_attn_dilated_indices(B: int, H: int, N: int, window: int, dilation: int,
                                k: Optional[int] = None, device="cuda",
                                idx: Optional[torch.Tensor] = None,
                                profile: Optional[Profile] = None) -> torch.Tensor:
    """idx [B,H,N,k]: (i + t*dilation) mod N for t < window, then -1."""
    if k is None:
        k = window
    if idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=device)
    _tensor(idx, "idx")
    if idx.dtype != torch.int32 or tuple(idx.shape) != (B, H, N, k):
        raise ValueError(f"idx must be int32 [B, H, N, k] = {(B, H, N, k)}")
    st = load_library().sparse_attn_dilated_indices(sa_dims(B, H, N, 0), window, dilation,
                                                    _dev(idx, "idx"), k,
                                                    _options(None, profile), _stream(idx))
    _check(st, "sparse_attn_dilated_indices")
    return idx


def sparse_attn_band_indices_per_batch(H: int, N: int, radii: torch.Tensor,
                                       k: Optional[int] = None,
                                       idx: Optional[torch.Tensor] = None,
                                       profile: Optional[Profile] = None) -> torch.Tensor:
    """idx [B,H,N,k] with B = len(radii): sample b's rows are its band of
    radius radii[b] (an int32 tensor on the GPU)."""
    _tensor(radii, "radii")
    if radii.dtype != torch.int32 or radii.dim() != 1:
        raise ValueError("radii must be a 1-D int32 tensor")
    B = radii.shape[0]
    if k is None:
        k = 2 * int(radii.max().item()) + 1
    if idx is None:
        idx = torch.empty((B, H, N, k), dtype=torch.int32, device=radii.device)
    _tensor(idx, "idx")
    if idx.dtype != torch.int32 or tuple(idx.shape) != (B, H, N, k):
        raise ValueError(f"idx must be int32 [B, H, N, k] = {(B, H, N, k)}")
    if idx.device != radii.device:
        raise ValueError("idx and radii must be on one device")
    st = load_library().sparse_attn_band_indices_per_batch(
        sa_dims(B, H, N, 0), _dev(radii, "radii"), _dev(idx, "idx"), k,
        _options(None, profile), _stream(idx))
    _check(st, "sparse_attn_band_indices_per_batch")
    return idx


def sparse_attn_bwd(Q, K, V, dO, idx, Pq=None, Pk=None, scorer_grad: bool = True,
                    score_scale: Optional[float] = None, softmax_scale: Optional[float] = None,
                    workspace: Optional[torch.Tensor] = None,
                    profile: Optional[Profile] = None, parts: str = "auto"):
    """Gradients of the forward for index sets idx: returns (dQ, dK, dV) in
    fp32, plus (dPq, dPk) when scorer_grad (the straight-through gradient
    of the scorer; Pq, Pk required).  parts: "auto", "whole" or "split",
    the layout of the library's row and key passes (same results)."""
    _check_qkv(Q, K, V, dO)
    _tensor(idx, "idx")
    if idx.dim() != 4:
        raise ValueError("idx must be [B, H, N, k]")
    k = idx.shape[-1]
    _check_idx(idx, Q, k)
    B, H, N, D = Q.shape
    d_proj = 16
    if scorer_grad:
        d_proj = _check_proj(Pq, Pk, Q)
    sscale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    ascale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    lib = load_library()
    if workspace is None:
        n = int(lib.sparse_attn_bwd_workspace_size(_dims(Q), d_proj, k, int(scorer_grad),
                                                   _options(None, None, parts)))
        if n == 0:
            raise SparseAttnError(-3, "sparse_attn_bwd_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=Q.device)
    _check_workspace(workspace, Q)
    f32 = dict(dtype=torch.float32, device=Q.device)
    dQ, dK, dV = (torch.empty(B, H, N, D, **f32) for _ in range(3))
    dPq = torch.empty(D, d_proj, **f32) if scorer_grad else None
    dPk = torch.empty(D, d_proj, **f32) if scorer_grad else None
    st = lib.sparse_attn_bwd(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(Pq, "Pq") if scorer_grad else None,
        _dev(Pk, "Pk") if scorer_grad else None, _dev(dO, "dO"), _dev(idx, "idx"), _dims(Q),
        d_proj, k, sscale, ascale, _dtype_code(Q), _dev(dQ, "dQ"), _dev(dK, "dK"),
        _dev(dV, "dV"), _dev(dPq, "dPq") if scorer_grad else None,
        _dev(dPk, "dPk") if scorer_grad else None, _dev(workspace, "workspace"),
        workspace.numel(), _options(None, profile, parts), _stream(Q))
    _check(st, "sparse_attn_bwd")
    return (dQ, dK, dV, dPq, dPk) if scorer_grad else (dQ, dK, dV)


def _block_workspace(Q, d_proj: int, block: int, kb: int) -> torch.Tensor:
    B, H, N, D = Q.shape
    n = int(load_library().sparse_attn_block_workspace_size(sa_dims(B, H, N, D), d_proj, block,
                                                            kb))
    if n == 0:
        raise SparseAttnError(-3, "sparse_attn_block_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=Q.device)


def sparse_attn_block_topk(Q, K, Pq, Pk, block: int, kb: int, causal: bool = False,
                           score_scale: Optional[float] = None,
                           idx: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           profile: Optional[Profile] = None) -> torch.Tensor:
    """idx [B,H,N,kb*block]: the keys of each query's kb best key blocks."""
    _check_qkv(Q, K)
    d_proj = _check_proj(Pq, Pk, Q)
    B, H, N, D = Q.shape
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    if idx is None:
        idx = torch.empty((B, H, N, kb * block), dtype=torch.int32, device=Q.device)
    _check_idx(idx, Q, kb * block)
    if workspace is None:
        workspace = _block_workspace(Q, d_proj, block, kb)
    _check_workspace(workspace, Q)
    st = load_library().sparse_attn_block_topk(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj, block, kb,
        int(causal), scale, _dtype_code(Q), _dev(idx, "idx"), _dev(workspace, "workspace"),
        workspace.numel(), _options(None, profile), _stream(Q))
    _check(st, "sparse_attn_block_topk")
    return idx


def sparse_attn_block_scores_dump(Q, K, Pq, Pk, block: int, row_begin: int, row_count: int,
                                  score_scale: Optional[float] = None,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S [B,H,row_count,ceil(N/block)] fp32: the block scores the block
    selection ranks."""
    _check_qkv(Q, K)
    d_proj = _check_proj(Pq, Pk, Q)
    B, H, N, D = Q.shape
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    NB = (N + block - 1) // block
    S = torch.empty((B, H, row_count, NB), dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = _block_workspace(Q, d_proj, block, 1)
    _check_workspace(workspace, Q)
    st = load_library().sparse_attn_block_scores_dump(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj, block,
        scale, _dtype_code(Q), row_begin, row_count, _dev(S, "S"), _dev(workspace, "workspace"),
        workspace.numel(), None, _stream(Q))
    _check(st, "sparse_attn_block_scores_dump")
    return S


class DecodeCache:
    """Caller-owned caches of the decode path: K and V caches [B,H,Ncap,D]
    of the model's dtype and the k_low cache [B,H,Ncap,d_proj] fp32, plus
    the decode workspace.  append() writes new keys (and values) at the
    current length; step() runs one query per (b, h) over the cached keys."""

    def __init__(self, B: int, H: int, Ncap: int, D: int, Pq, Pk, k: int,
                 dtype=torch.bfloat16, device="cuda"):
        _tensor(Pq, "Pq")
        _like(Pk, Pq, "Pk", "Pq")
        if Pq.dim() != 2 or Pq.shape[0] != D or Pq.dtype != dtype:
            raise ValueError(f"Pq, Pk must be [{D}, d_proj] of {dtype}")
        self.B, self.H, self.Ncap, self.D, self.k = B, H, Ncap, D, k
        self.d_proj = int(Pq.shape[1])
        self.Pq, self.Pk = Pq, Pk
        self.dtype = dtype
        self.K = torch.zeros(B, H, Ncap, D, dtype=dtype, device=device)
        self.V = torch.zeros(B, H, Ncap, D, dtype=dtype, device=device)
        self.klow = torch.zeros(B, H, Ncap, self.d_proj, dtype=torch.float32, device=device)
        self.counts = torch.zeros(B, H, Ncap, dtype=torch.int32, device=device)
        n = int(load_library().sparse_attn_decode_workspace_size(sa_dims(B, H, Ncap, D),
                                                                 self.d_proj, k))
        if n == 0:
            raise SparseAttnError(-3, "sparse_attn_decode_workspace_size")
        self.workspace = torch.empty(n, dtype=torch.uint8, device=device)
        self.len = 0

    def append(self, K_new, V_new, profile: Optional[Profile] = None) -> None:
        """Write T new keys and values [B,H,T,D] at rows len .. len+T-1."""
        _tensor(K_new, "K_new")
        if K_new.dim() != 4 or tuple(K_new.shape[:2]) != (self.B, self.H) or \
                K_new.shape[3] != self.D or K_new.dtype != self.dtype:
            raise ValueError("K_new must be [B, H, T, D] of the cache's dtype")
        _like(V_new, K_new, "V_new", "K_new")
        T = int(K_new.shape[2])
        if self.len + T > self.Ncap:
            raise ValueError("the cache is full")
        st = load_library().sparse_attn_decode_append_keys(
            _dev(K_new, "K_new"), _dev(self.Pk, "Pk"), sa_dims(self.B, self.H, T, self.D),
            self.d_proj, _dtype_code(K_new), _dev(self.klow, "klow"), self.Ncap, self.len,
            _options(None, profile), _stream(K_new))
        _check(st, "sparse_attn_decode_append_keys")
        self.K[:, :, self.len:self.len + T] = K_new
        self.V[:, :, self.len:self.len + T] = V_new
        self.len += T

    def step_noalloc(self, q, O: torch.Tensor, idx: Optional[torch.Tensor] = None,
                     count: bool = False, score_scale: Optional[float] = None,
                     softmax_scale: Optional[float] = None):
        """step() through sparse_attn_decode_noalloc: the library's own
        device-resident workspace, no allocation (O must be given)."""
        _tensor(q, "q")
        if tuple(q.shape) != (self.B, self.H, 1, self.D) or q.dtype != self.dtype:
            raise ValueError(f"q must be [B, H, 1, D] = {(self.B, self.H, 1, self.D)} "
                             f"of {self.dtype}")
        _like(O, q, "O", "q")
        if idx is not None:
            _tensor(idx, "idx")
            if idx.dtype != torch.int32 or tuple(idx.shape) != (self.B, self.H, self.k):
                raise ValueError(f"idx must be int32 [B, H, k] = {(self.B, self.H, self.k)}")
        if self.len < 1:
            raise ValueError("the cache is empty")
        sscale = default_score_scale(self.d_proj) if score_scale is None else float(score_scale)
        ascale = default_softmax_scale(self.D) if softmax_scale is None else float(softmax_scale)
        st = load_library().sparse_attn_decode_noalloc(
            _dev(q, "q"), _dev(self.K, "K"), _dev(self.V, "V"), _dev(self.klow, "klow"),
            _dev(self.Pq, "Pq"), sa_dims(self.B, self.H, self.Ncap, self.D), self.d_proj,
            self.len, self.k, sscale, ascale, _dtype_code(q), _dev(O, "O"),
            None if idx is None else _dev(idx, "idx"),
            _dev(self.counts, "counts") if count else None, _stream(q))
        _check(st, "sparse_attn_decode_noalloc")
        return (O, idx) if idx is not None else O

    def step(self, q, score_scale: Optional[float] = None,
             softmax_scale: Optional[float] = None, O: Optional[torch.Tensor] = None,
             idx: Optional[torch.Tensor] = None, count: bool = False,
             profile: Optional[Profile] = None):
        """O [B,H,1,D] (and idx [B,H,k]) of one query per (b, h) over the
        cached keys 0 .. len-1."""
        _tensor(q, "q")
        if tuple(q.shape) != (self.B, self.H, 1, self.D) or q.dtype != self.dtype:
            raise ValueError(f"q must be [B, H, 1, D] = {(self.B, self.H, 1, self.D)} "
                             f"of {self.dtype}")
        if self.len < 1:
            raise ValueError("the cache is empty")
        sscale = default_score_scale(self.d_proj) if score_scale is None else float(score_scale)
        ascale = default_softmax_scale(self.D) if softmax_scale is None else float(softmax_scale)
        if O is None:
            O = torch.empty_like(q)
        _like(O, q, "O", "q")
        if idx is not None:
            _tensor(idx, "idx")
            if idx.dtype != torch.int32 or tuple(idx.shape) != (self.B, self.H, self.k):
                raise ValueError(f"idx must be int32 [B, H, k] = {(self.B, self.H, self.k)}")
        st = load_library().sparse_attn_decode(
            _dev(q, "q"), _dev(self.K, "K"), _dev(self.V, "V"), _dev(self.klow, "klow"),
            _dev(self.Pq, "Pq"), sa_dims(self.B, self.H, self.Ncap, self.D), self.d_proj,
            self.len, self.k, sscale, ascale, _dtype_code(q), _dev(O, "O"),
            None if idx is None else _dev(idx, "idx"),
            _dev(self.counts, "counts") if count else None,
            _dev(self.workspace, "workspace"), self.workspace.numel(),
            _options(None, profile), _stream(q))
        _check(st, "sparse_attn_decode")
        return (O, idx) if idx is not None else O


def sparse_attn_scores_dump(Q, K, Pq, Pk, row_begin: int, row_count: int,
                            causal: bool = False, score_scale: Optional[float] = None,
                            S: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S [B,H,row_count,N] fp32: the exact scores the selection uses."""
    _check_qkv(Q, K)
    d_proj = _check_proj(Pq, Pk, Q)
    B, H, N, D = Q.shape
    scale = default_score_scale(d_proj) if score_scale is None else float(score_scale)
    if S is None:
        S = torch.empty((B, H, row_count, N), dtype=torch.float32, device=Q.device)
    _tensor(S, "S")
    if S.dtype != torch.float32 or tuple(S.shape) != (B, H, row_count, N):
        raise ValueError(f"S must be float32 [B, H, row_count, N] = {(B, H, row_count, N)}")
    if workspace is None:
        workspace = allocate_workspace(Q, d_proj, 1, causal)
    _check_workspace(workspace, Q)
    st = load_library().sparse_attn_scores_dump(
        _dev(Q, "Q"), _dev(K, "K"), _dev(Pq, "Pq"), _dev(Pk, "Pk"), _dims(Q), d_proj,
        int(causal), scale, _dtype_code(Q), row_begin, row_count, _dev(S, "S"),
        _dev(workspace, "workspace"), workspace.numel(), None, _stream(Q))
    _check(st, "sparse_attn_scores_dump")
    return S


def sparse_attn_check_status(stream: Optional[int] = None) -> int:
    """Synchronizes and returns SA_OK or SA_ERR_DEVICE_INDEX (clearing it)."""
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    return int(load_library().sparse_attn_check_status(s))


STAT_KEYS = ("fallback_queries", "overflow_queries", "candidates", "rescored", "queries",
             "retried", "margin_violations", "wide_queries")


def sparse_attn_workspace_stats(workspace: torch.Tensor) -> dict:
    out = (ctypes.c_int64 * len(STAT_KEYS))()
    n = load_library().sparse_attn_workspace_stats(
        _dev(workspace, "workspace"), workspace.numel(), out, len(STAT_KEYS),
        _stream(workspace))
    if n < 0:
        raise SparseAttnError(n, "sparse_attn_workspace_stats")
    return {kk: int(out[i]) for i, kk in enumerate(STAT_KEYS[:n])}


__all__ = [
    "sa_dims", "sa_options", "SparseAttnError", "load_library", "status_string", "LIB_PATH",
    "EXPORTS", "Profile", "sparse_attn_workspace_size", "allocate_workspace",
    "sparse_attn_scores_topk", "sparse_attn_gather", "sparse_attn_fwd",
    "sparse_attn_band_indices", "sparse_attn_scores_dump", "sparse_attn_check_status",
    "sparse_attn_workspace_stats", "default_score_scale", "default_softmax_scale",
    "sparse_attn_scores_topk_smoothed", "sparse_attn_dilated_indices",
    "sparse_attn_band_indices_per_batch", "DecodeCache", "sparse_attn_block_topk",
    "sparse_attn_block_scores_dump", "sparse_attn_bwd",
]
