"""The C-ABI library without a GPU: it builds, loads, exports every symbol the
header declares, and rejects bad arguments on the host before touching HIP.

Only argument combinations that fail host-side validation are passed here
(fake but 16-byte-aligned addresses never reach a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import dynamic_top_sparse_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.LIB_PATH):
        from dynamic_top_sparse_amd import build
        build.build()
    return sa.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert _declared() == sorted(sa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


D = sa.sa_dims
A = 0x100000  # a 16-byte-aligned fake address: never dereferenced in these tests


def test_filter_dtype_option(lib):
    assert lib.sparse_attn_get_filter_dtype() == 2          # fp16 by default
    assert lib.sparse_attn_set_filter_dtype(0) == -3        # fp32 is not a filter type
    assert lib.sparse_attn_set_filter_dtype(1) == 0
    assert lib.sparse_attn_get_filter_dtype() == 1
    assert lib.sparse_attn_set_filter_dtype(2) == 0


def test_status_strings(lib):
    for code in range(0, -8, -1):
        assert lib.sparse_attn_status_string(code)
    assert sa.status_string(-5) == "workspace too small"


def test_workspace_size_arithmetic(lib):
    d = D(1, 32, 131072, 128)
    one = lib.sparse_attn_workspace_size_for_chunk(d, 64, 512, 0, 1, 0, 1)
    two = lib.sparse_attn_workspace_size_for_chunk(d, 64, 512, 0, 1, 0, 2)
    eight = lib.sparse_attn_workspace_size(d, 64, 512, 0, 1, 0)
    assert 0 < one < two < eight
    assert eight == lib.sparse_attn_workspace_size_for_chunk(d, 64, 512, 0, 1, 0, 8)
    # idx room: N*k*4 bytes per head of the chunk
    with_idx = lib.sparse_attn_workspace_size_for_chunk(d, 64, 512, 0, 1, 1, 1)
    assert with_idx - one >= 131072 * 512 * 4
    # unsupported arguments give 0
    assert lib.sparse_attn_workspace_size(D(1, 1, 1024, 96), 16, 32, 0, 0, 0) == 0
    assert lib.sparse_attn_workspace_size(D(1, 1, 1024, 64), 24, 32, 0, 0, 0) == 0
    assert lib.sparse_attn_workspace_size(D(1, 1, 1024, 64), 16, 4096, 0, 0, 0) == 0
    assert lib.sparse_attn_workspace_size(D(0, 1, 1024, 64), 16, 32, 0, 0, 0) == 0


def _topk(lib, Q=A, K=A, Pq=A, Pk=A, d=D(1, 1, 1024, 64), dp=16, k=32, causal=0, scale=0.25,
          dtype=0, idx=A, ws=A, ws_bytes=0):
    return lib.sparse_attn_scores_topk(Q, K, Pq, Pk, d, dp, k, causal, scale, dtype, idx, ws,
                                       ws_bytes, None)


def test_scores_topk_validation(lib):
    assert _topk(lib, Q=None) == -1
    assert _topk(lib, idx=None) == -1
    assert _topk(lib, d=D(1, 1, 0, 64)) == -2
    assert _topk(lib, k=0) == -2
    assert _topk(lib, d=D(1, 1, 2**21, 64), k=1024) == -2     # N*k >= 2^31
    assert _topk(lib, k=4096) == -3
    assert _topk(lib, d=D(1, 1, 1024, 80)) == -3
    assert _topk(lib, dp=8) == -3
    assert _topk(lib, dtype=2) == -3
    assert _topk(lib, scale=0.0) == -2
    assert _topk(lib, scale=float("nan")) == -2
    assert _topk(lib, Q=A + 4) == -4
    assert _topk(lib, ws=A + 8) == -4
    assert _topk(lib, ws_bytes=1024) == -5                    # workspace too small


def test_gather_fwd_band_dump_validation(lib):
    d = D(1, 2, 256, 64)
    assert lib.sparse_attn_gather(A, A, None, A, 8, d, 0.1, 0, A, None) == -1
    assert lib.sparse_attn_gather(A, A, A, A, 0, d, 0.1, 0, A, None) == -2
    assert lib.sparse_attn_gather(A, A, A, A, 8, D(1, 2, 256, 32), 0.1, 0, A, None) == -3
    assert lib.sparse_attn_gather(A, A, A, A + 4, 8, d, 0.1, 0, A, None) == -4
    assert lib.sparse_attn_gather(A, A, A, A, 8, d, float("inf"), 0, A, None) == -2
    assert lib.sparse_attn_fwd(A, A, A, A, A, d, 16, 8, 0, 0.25, 0.1, 0, None, None, A, 1 << 30,
                               None) == -1
    assert lib.sparse_attn_fwd(A, A, A, A, A, d, 16, 8, 0, 0.25, 0.1, 1, A, A + 2, A, 1 << 30,
                               None) == -4
    assert lib.sparse_attn_fwd(A, A, A, A, A, d, 16, 8, 0, 0.25, 0.1, 1, A, None, A, 64,
                               None) == -5
    assert lib.sparse_attn_band_indices(d, -1, 3, A, 5, None) == -2
    assert lib.sparse_attn_band_indices(d, 1, 3, None, 5, None) == -1
    assert lib.sparse_attn_band_indices(d, 1, 3, A + 4, 5, None) == -4
    assert lib.sparse_attn_scores_dump(A, A, A, A, d, 16, 0, 0.25, 0, 250, 7, A, A, 1 << 30,
                                       None) == -2               # rows past N
    assert lib.sparse_attn_scores_dump(A, A, A, A, d, 16, 0, 0.25, 0, -1, 1, A, A, 1 << 30,
                                       None) == -2
    assert lib.sparse_attn_scores_dump(A, A, A, A, d, 16, 0, 0.25, 0, 0, 1, A, A, 16,
                                       None) == -5
    out = (ctypes.c_int64 * 5)()
    assert lib.sparse_attn_workspace_stats(None, 1024, out, 5, None) == -1
    assert lib.sparse_attn_workspace_stats(A, 8, out, 5, None) == -5


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    p = torch.zeros(64, 16)
    with pytest.raises((ValueError, RuntimeError)):
        sa.sparse_attn_scores_topk(q, q, p, p, 4)
    with pytest.raises((ValueError, RuntimeError)):
        sa.sparse_attn_gather(q, q, q, torch.zeros(1, 1, 64, 4, dtype=torch.int32))
