"""The seeded input generators: determinism, shapes, dtypes, distributions."""
import torch

from dynamic_top_sparse_amd import workloads as W


def test_five_workloads_have_the_stated_shapes():
    t = W.WORKLOADS
    assert (t["tiny_fp32"].B, t["tiny_fp32"].H, t["tiny_fp32"].N, t["tiny_fp32"].D) == (1, 1, 1024, 64)
    assert (t["tiny_fp32"].d_proj, t["tiny_fp32"].k) == (16, 32)
    assert t["band_fp32"].mode == "band" and t["band_fp32"].window == 64
    assert (t["bf16_32k"].H, t["bf16_32k"].N, t["bf16_32k"].k) == (32, 32768, 256)
    h = t["headline_128k"]
    assert (h.B, h.H, h.N, h.D, h.d_proj, h.k, h.causal) == (1, 32, 131072, 128, 64, 512, False)
    c = t["causal_mixture"]
    assert (c.B, c.H, c.N, c.causal, c.dist) == (4, 8, 65536, True, "mixture")


def test_generation_is_deterministic_and_typed():
    w = W.get("tiny_fp32")
    a, b = W.make_inputs(w, 0), W.make_inputs(w, 0)
    for name in ("Q", "K", "V", "Pq", "Pk"):
        assert torch.equal(a[name], b[name])
        assert a[name].dtype == torch.float32 and a[name].is_contiguous()
    assert a["Pq"].shape == (64, 16)
    c = W.make_inputs(w, 1)
    assert not torch.equal(a["Q"], c["Q"])


def test_bf16_workload_and_projection_scale():
    w = W.get("bf16_32k", N=2048, H=2)
    x = W.make_inputs(w, 0)
    assert x["Q"].dtype == torch.bfloat16 and x["Q"].shape == (1, 2, 2048, 128)
    std = x["Pq"].float().std().item()
    assert abs(std - 128 ** -0.5) < 0.01


def test_mixture_rows_cluster_around_shared_centres():
    w = W.get("causal_mixture", B=1, H=1, N=4096)
    x = W.make_inputs(w, 0)
    q = x["Q"].float()[0, 0]
    # nearest-neighbour distance is ~ noise scale, far below N(0,1) spacing
    d = torch.cdist(q[:256], q[256:2304]).min(dim=1).values
    assert d.median().item() < 0.3 * (2 * 128) ** 0.5
    assert x["V"].float().std().item() > 0.9


def test_band_workload_has_no_projection():
    x = W.make_inputs(W.get("band_fp32", H=1, N=256), 0)
    assert set(x) == {"Q", "K", "V"}
