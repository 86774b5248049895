"""sparse_attn_decode_noalloc: the decode step with the library's own
device-resident workspace (for callers that cannot allocate) gives exactly
the results of sparse_attn_decode with a caller workspace, on two calls in a
row, the second smaller; a call too large for the array is refused on the
host."""
import ctypes

import numpy as np
import pytest
import torch

import dynamic_top_sparse_amd as sa
from dynamic_top_sparse_amd import workloads as W

pytestmark = pytest.mark.gpu


def _case(B, H, N, D, dp, k, length, seed, dtype="bf16"):
    w = W.Workload("noalloc", B, H, N, D, dtype, d_proj=dp, k=k, causal=True)
    x = W.make_inputs(w, seed)
    g = {n: t.cuda() for n, t in x.items()}
    cache = sa.DecodeCache(B, H, N, D, g["Pq"], g["Pk"], k, dtype=w.torch_dtype)
    cache.append(g["K"][:, :, :length].contiguous(), g["V"][:, :, :length].contiguous())
    q = g["Q"][:, :, length - 1:length].contiguous()
    return cache, q


def test_noalloc_decode_equals_decode_twice():
    cases = [(2, 8, 8192, 128, 64, 256, 8000, 1),     # the larger call first
             (1, 3, 3000, 64, 16, 40, 2999, 2)]       # then a smaller one
    for (B, H, N, D, dp, k, length, seed) in cases:
        cache, q = _case(B, H, N, D, dp, k, length, seed)
        O1 = torch.empty_like(q)
        i1 = torch.empty(B, H, k, dtype=torch.int32, device="cuda")
        cache.step(q, O=O1, idx=i1)
        O2 = torch.full_like(q, float("nan"))
        i2 = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
        cache.step_noalloc(q, O2, idx=i2)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2), (B, H, N)
        assert torch.equal(O1, O2), (B, H, N)


def test_noalloc_refuses_sizes_beyond_its_array():
    lib = sa.load_library()
    cap = lib.sparse_attn_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    d = sa.sa_dims(4, 16, 200000, 128)            # 64 heads x 200K scores: 51 MB
    assert lib.sparse_attn_decode_workspace_size(d, 64, 512) > cap
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    p = t.data_ptr()
    st = lib.sparse_attn_decode_noalloc(p, p, p, p, p, d, 64, 100, 512, 0.125, 0.088, 1, p,
                                        None, None, None)
    assert st == -5                                # SA_ERR_WORKSPACE, nothing enqueued
