"""The seeded generators: shapes, dtypes, reproducibility and the skewed-workload recipe."""
import numpy as np
import torch

import workloads


def test_shapes_and_reproducible():
    cfg = workloads.get("tiny_fp32")
    a = workloads.make_layer_inputs(cfg)
    b = workloads.make_layer_inputs(cfg)
    assert a["x"].shape == (64, 256) and a["x"].dtype == torch.float32
    assert a["w_gate"].shape == (17, 128, 256) and a["w_down"].shape == (17, 256, 128)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    # different tensors and experts draw different numbers
    assert not torch.equal(a["w_gate"][0], a["w_gate"][1])
    assert not torch.equal(a["w_gate"][0], a["w_up"][0])
    assert abs(a["w_gate"].std().item() - 0.02) < 1e-3


def test_fp8_weights_stored_form():
    cfg = workloads.get("prefill_fp8").replace(T=4, hidden=256, inter=128, E=4, K=2, G=2, M=1)
    d = workloads.make_layer_inputs(cfg)
    assert d["w_gate"].dtype == torch.float8_e4m3fn and d["s_gate"].shape == (5, 1, 2)
    assert d["s_down"].shape == (5, 2, 1)
    deq = d["w_gate"][0, :, :128].float() * d["s_gate"][0, 0, 0]
    assert 0.005 < deq.std().item() < 0.04


def test_skew_recipe():
    cfg = workloads.get("skewed_bf16").replace(T=8, hidden=64, E=16, K=2, G=4, M=2)
    x = workloads.make_tokens(cfg)
    w = workloads.make_router(cfg)
    assert torch.all(x[:, 0] == 1.0)
    assert torch.all(w[:8, 0] == 2.0) and torch.all(w[8:, 0] == 0.0)


def test_sample_rows():
    r = workloads.sample_rows(8192, 512)
    assert r.shape == (512,) and torch.all(r[1:] > r[:-1])
    assert torch.equal(r, workloads.sample_rows(8192, 512))


def test_topk_with_loads_histogram_and_distinct():
    loads = [0, 3, 5, 5, 5, 5, 2]
    idx = workloads.topk_with_loads(5, 5, loads)
    assert idx.shape == (5, 5) and idx.dtype == torch.int32
    assert np.bincount(idx.numpy().ravel(), minlength=7).tolist() == loads
    assert all(len(set(row.tolist())) == 5 for row in idx)
