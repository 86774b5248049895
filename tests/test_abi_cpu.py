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


def test_options_and_profile_record(lib):
    """Options are per call: an unknown filter type is refused on the host;
    a timing record is created, read empty and destroyed without a GPU."""
    bad = sa.sa_options(0, None)                           # fp32 is not a filter type
    assert _topk(lib, opts=ctypes.byref(bad)) == -3
    assert lib.sparse_attn_fwd(A, A, A, A, A, D(1, 2, 256, 64), 16, 8, 0, 0.25, 0.1, 1, A,
                               None, A, 1 << 30, ctypes.byref(bad), None) == -3
    prof = lib.sparse_attn_profile_create()
    assert prof
    out = (sa.sa_kernel_time * 4)()
    assert lib.sparse_attn_profile_read(prof, out, 4) == 0
    assert lib.sparse_attn_profile_read(None, out, 4) == -1
    lib.sparse_attn_profile_destroy(prof)
    lib.sparse_attn_profile_destroy(None)


def test_header_has_no_process_wide_setters():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in re.findall(r"\b(sparse_attn_\w+)\s*\(", text):
        assert "set_" not in name and "enable" not in name, name


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


def test_gather_ws_size_and_validation(lib):
    # the key-range path applies past N = 8192: 36 B of segment starts and 4 B of
    # list per row, a count, and one head's partials (8 ranges x (D + 4) floats)
    assert lib.sparse_attn_gather_workspace_size(D(1, 2, 8192, 128), 64, 1) == 0
    n = lib.sparse_attn_gather_workspace_size(D(1, 2, 8200, 128), 64, 1)
    rows = 2 * 8200
    assert n >= rows * 40 + 8200 * 8 * 132 * 4
    assert n < rows * 40 + 8200 * 8 * 132 * 4 + 4 * 256
    assert lib.sparse_attn_gather_workspace_size(D(1, 2, 8200, 96), 64, 1) == 0
    assert lib.sparse_attn_gather_workspace_size(D(1, 2, 8200, 128), 64, 2) == 0
    assert lib.sparse_attn_gather_workspace_size(D(1, 2**17, 8200, 64), 1, 1) > 0
    assert lib.sparse_attn_gather_workspace_size(D(1, 2**18, 8200, 64), 1, 1) == 0   # > 2^31 rows
    big = D(1, 2, 8200, 128)
    g = lambda **kw: lib.sparse_attn_gather_ws(
        kw.get("Q", A), A, A, kw.get("idx", A), kw.get("k", 64), kw.get("d", big),
        kw.get("scale", 0.1), kw.get("dtype", 1), A, kw.get("ws", A), kw.get("ws_bytes", n),
        None, None)
    assert g(Q=None) == -1
    assert g(k=0) == -2
    assert g(scale=float("nan")) == -2
    assert g(dtype=2) == -3
    assert g(idx=A + 4) == -4
    assert g(ws=None) == -1                      # the key-range path needs its workspace
    assert g(ws=A + 8) == -4
    assert g(ws_bytes=n - 1) == -5


def _topk(lib, Q=A, K=A, Pq=A, Pk=A, d=D(1, 1, 1024, 64), dp=16, k=32, causal=0, scale=0.25,
          dtype=0, idx=A, ws=A, ws_bytes=0, opts=None):
    return lib.sparse_attn_scores_topk(Q, K, Pq, Pk, d, dp, k, causal, scale, dtype, idx, ws,
                                       ws_bytes, opts, None)


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
    assert lib.sparse_attn_gather(A, A, None, A, 8, d, 0.1, 0, A, None, None) == -1
    assert lib.sparse_attn_gather(A, A, A, A, 0, d, 0.1, 0, A, None, None) == -2
    assert lib.sparse_attn_gather(A, A, A, A, 8, D(1, 2, 256, 32), 0.1, 0, A, None, None) == -3
    assert lib.sparse_attn_gather(A, A, A, A + 4, 8, d, 0.1, 0, A, None, None) == -4
    assert lib.sparse_attn_gather(A, A, A, A, 8, d, float("inf"), 0, A, None, None) == -2
    assert lib.sparse_attn_fwd(A, A, A, A, A, d, 16, 8, 0, 0.25, 0.1, 0, None, None, A, 1 << 30,
                               None, None) == -1
    assert lib.sparse_attn_fwd(A, A, A, A, A, d, 16, 8, 0, 0.25, 0.1, 1, A, A + 2, A, 1 << 30,
                               None, None) == -4
    assert lib.sparse_attn_fwd(A, A, A, A, A, d, 16, 8, 0, 0.25, 0.1, 1, A, None, A, 64,
                               None, None) == -5
    assert lib.sparse_attn_band_indices(d, -1, 3, A, 5, None, None) == -2
    assert lib.sparse_attn_band_indices(d, 1, 3, None, 5, None, None) == -1
    assert lib.sparse_attn_band_indices(d, 1, 3, A + 4, 5, None, None) == -4
    assert lib.sparse_attn_scores_dump(A, A, A, A, d, 16, 0, 0.25, 0, 250, 7, A, A, 1 << 30,
                                       None, None) == -2         # rows past N
    assert lib.sparse_attn_scores_dump(A, A, A, A, d, 16, 0, 0.25, 0, -1, 1, A, A, 1 << 30,
                                       None, None) == -2
    assert lib.sparse_attn_scores_dump(A, A, A, A, d, 16, 0, 0.25, 0, 0, 1, A, A, 16,
                                       None, None) == -5
    out = (ctypes.c_int64 * 5)()
    assert lib.sparse_attn_workspace_stats(None, 1024, out, 5, None) == -1
    assert lib.sparse_attn_workspace_stats(A, 8, out, 5, None) == -5


def _qkv(B=1, H=2, N=64, D=64, dtype=None):
    import torch
    dtype = dtype or torch.float32
    return [torch.zeros(B, H, N, D, dtype=dtype) for _ in range(3)]


@pytest.mark.parametrize("what", ["K_shape", "V_shape", "K_dtype", "O_shape", "O_dtype",
                                  "Pq_rows", "Pk_shape", "P_dtype", "idx_dtype", "idx_shape",
                                  "idx_k"])
def test_binding_rejects_mismatched_tensors(what):
    """Every tensor is checked against Q before anything reaches the library:
    a smaller K or V, a mixed dtype, a wrong-width Pk or a short idx would
    otherwise be read or written past its end by the kernels."""
    import torch
    Q, K, V = _qkv()
    Pq = torch.zeros(64, 16)
    Pk = torch.zeros(64, 16)
    idx = torch.zeros(1, 2, 64, 8, dtype=torch.int32)
    O = None
    if what == "K_shape":
        K = torch.zeros(1, 2, 32, 64)
    elif what == "V_shape":
        V = torch.zeros(1, 1, 64, 64)
    elif what == "K_dtype":
        K = K.to(torch.bfloat16)
    elif what == "O_shape":
        O = torch.zeros(1, 2, 64, 32)
    elif what == "O_dtype":
        O = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    elif what == "Pq_rows":
        Pq = torch.zeros(32, 16)
    elif what == "Pk_shape":
        Pk = torch.zeros(64, 32)
    elif what == "P_dtype":
        Pq, Pk = Pq.to(torch.bfloat16), Pk.to(torch.bfloat16)
    elif what == "idx_dtype":
        idx = idx.to(torch.int16)
    elif what == "idx_shape":
        idx = torch.zeros(1, 2, 63, 8, dtype=torch.int32)
    elif what == "idx_k":
        idx = torch.zeros(1, 2, 64, 9, dtype=torch.int32)
    with pytest.raises(ValueError):
        if what.startswith("idx"):
            sa.sparse_attn_scores_topk(Q, K, Pq, Pk, 8, idx=idx, workspace=torch.zeros(1, dtype=torch.uint8))
        elif what in ("V_shape", "O_shape", "O_dtype"):
            sa.sparse_attn_fwd(Q, K, V, Pq, Pk, 8, O=O, workspace=torch.zeros(1, dtype=torch.uint8))
        else:
            sa.sparse_attn_fwd(Q, K, V, Pq, Pk, 8, workspace=torch.zeros(1, dtype=torch.uint8))
    if what.startswith("idx") or what in ("K_shape", "V_shape", "K_dtype", "O_shape"):
        with pytest.raises(ValueError):
            sa.sparse_attn_gather(Q, K, V, idx if what.startswith("idx") and what != "idx_k"
                                  else torch.zeros(1, 2, 63, 8, dtype=torch.int32), O=O)


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    p = torch.zeros(64, 16)
    with pytest.raises((ValueError, RuntimeError)):
        sa.sparse_attn_scores_topk(q, q, p, p, 4)
    with pytest.raises((ValueError, RuntimeError)):
        sa.sparse_attn_gather(q, q, q, torch.zeros(1, 1, 64, 4, dtype=torch.int32))


def test_index_variant_validation(lib):
    d = D(2, 3, 100, 64)
    assert lib.sparse_attn_dilated_indices(d, 4, 2, None, 4, None, None) == -1
    assert lib.sparse_attn_dilated_indices(d, -1, 2, A, 4, None, None) == -2
    assert lib.sparse_attn_dilated_indices(d, 4, 0, A, 4, None, None) == -2
    assert lib.sparse_attn_dilated_indices(d, 4, 2, A + 4, 4, None, None) == -4
    assert lib.sparse_attn_band_indices_per_batch(d, None, A, 5, None, None) == -1
    assert lib.sparse_attn_band_indices_per_batch(d, A, A, 0, None, None) == -2
    sm = lib.sparse_attn_scores_topk_smoothed
    dd = D(1, 1, 1024, 64)
    assert sm(A, A, A, A, dd, 16, 0, 0, 0.25, 0.1, 0, A, A, 1 << 30, None, None) == -2
    assert sm(A, A, A, A, dd, 16, 2048, 0, 0.25, 0.1, 0, A, A, 1 << 30, None, None) == -3
    assert sm(A, A, A, A, dd, 16, 8, 0, 0.25, float("nan"), 0, A, A, 1 << 30, None, None) == -2
    assert sm(A, A, A, A, dd, 16, 8, 0, 0.25, 0.1, 0, None, A, 1 << 30, None, None) == -1
    assert sm(A, A, A, A, dd, 16, 8, 0, 0.25, 0.1, 0, A, A, 64, None, None) == -5


def test_decode_and_block_validation(lib):
    d = D(1, 2, 1000, 64)
    assert lib.sparse_attn_decode_workspace_size(d, 16, 32) > 1000 * 2 * 4
    assert lib.sparse_attn_decode_workspace_size(d, 24, 32) == 0
    ws = lib.sparse_attn_decode_workspace_size(d, 16, 32)
    dec = lib.sparse_attn_decode
    assert dec(A, A, A, A, A, d, 16, 0, 32, 0.25, 0.1, 0, A, None, None, A, ws, None, None) == -2
    assert dec(A, A, A, A, A, d, 16, 1001, 32, 0.25, 0.1, 0, A, None, None, A, ws, None, None) == -2
    assert dec(A, A, A, A, A, d, 16, 10, 32, 0.25, 0.1, 0, A, None, None, A, 16, None, None) == -5
    assert dec(A, A, None, A, A, d, 16, 10, 32, 0.25, 0.1, 0, A, None, None, A, ws, None, None) == -1
    app = lib.sparse_attn_decode_append_keys
    assert app(A, A, D(1, 2, 10, 64), 16, 0, A, 1000, 995, None, None) == -2   # past the cache
    assert app(A, A, D(1, 2, 10, 64), 16, 0, A, 1000, -1, None, None) == -2
    assert app(A, A, D(1, 2, 10, 64), 16, 0, A + 4, 1000, 0, None, None) == -4
    assert lib.sparse_attn_block_workspace_size(d, 16, 64, 4) > 0
    assert lib.sparse_attn_block_workspace_size(d, 16, 64, 33) == 0       # kb above 32
    assert lib.sparse_attn_block_workspace_size(d, 16, 512, 8) == 0       # kb*block above 2048
    bt = lib.sparse_attn_block_topk
    bws = lib.sparse_attn_block_workspace_size(d, 16, 64, 4)
    assert bt(A, A, A, A, d, 16, 0, 4, 0, 0.25, 0, A, A, bws, None, None) == -2
    assert bt(A, A, A, A, d, 16, 64, 33, 0, 0.25, 0, A, A, bws, None, None) == -3
    assert bt(A, A, A, A, d, 16, 64, 4, 0, 0.25, 0, A, A, 16, None, None) == -5
    assert bt(A, A, A, A, d, 16, 64, 4, 0, 0.25, 0, None, A, bws, None, None) == -1


def test_bwd_parts_option_sizes():
    """The backward's workspace query follows the parts option: the split
    layout needs room for the parts' records, an unknown value gets 0."""
    lib = sa.load_library()
    d = sa.sa_dims(1, 2, 4096, 128)
    size = {}
    for name, code in sa.BWD_PARTS.items():
        o = sa.sa_options(0, None, code)
        size[name] = lib.sparse_attn_bwd_workspace_size(d, 64, 64, 1, ctypes.byref(o))
    assert size["whole"] > 0 and size["split"] > size["whole"]
    assert size["auto"] == size["whole"]          # a small head runs whole
    assert lib.sparse_attn_bwd_workspace_size(d, 64, 64, 1, None) == size["auto"]
    # from 2^22 row elements per head (N = 32768 at D = 128) automatic splits
    big = sa.sa_dims(1, 2, 32768, 128)
    auto_big = lib.sparse_attn_bwd_workspace_size(big, 64, 256, 1, None)
    split_big = lib.sparse_attn_bwd_workspace_size(big, 64, 256, 1,
                                                   ctypes.byref(sa.sa_options(0, None, 2)))
    assert auto_big == split_big
    bad = sa.sa_options(0, None, 7)
    assert lib.sparse_attn_bwd_workspace_size(d, 64, 64, 1, ctypes.byref(bad)) == 0
    with pytest.raises(ValueError):
        sa._options(None, None, "halves")

