"""GPU parity of the individual stages through the C ABI, against the oracle.

Stage inputs come from the seeded generators (or the oracle), never from another
HIP stage, so every expected value is the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import (check_routing, config_of, log, oracle_route, route, permute,
                         workspace)

pytestmark = pytest.mark.gpu


def _router_inputs(cfg):
    return dict(x=workloads.make_tokens(cfg, 0, "cuda"), w_router=workloads.make_router(cfg, "cuda"),
                bias=workloads.make_bias(cfg, "cuda"))


@pytest.mark.parametrize("name,over", [
    ("tiny_fp32", {}),
    ("tiny_fp32", dict(T=1)),
    ("tiny_fp32", dict(T=67, bias="uniform", bias_range=0.05)),
    ("decode_bf16", {}),
    ("decode_bf16", dict(T=1)),
    ("decode_bf16", dict(T=333)),
    ("decode_bf16", dict(T=200, hidden=256, E=16, K=4, G=4, M=2)),       # E below one N tile
    ("decode_bf16", dict(T=257, G=1, M=1)),                             # no group limit
    ("decode_bf16", dict(T=300, G=64, M=3, K=8, topn=1)),               # 64 groups of 4
    ("prefill_bf16", {}),                                               # T = 8192
    ("skewed_bf16", {}),                                                # T = 16384, hot experts
])
def test_route_matches_oracle(name, over):
    cfg = workloads.get(name).replace(**over)
    log(f"route {name} {over}")
    d = _router_inputs(cfg)
    idx, gate = route(cfg, d)
    r = oracle_route(cfg, d)
    _, _, flipped = check_routing(cfg, r, idx, gate, where=name)
    ties = int(r.near_tie.sum())
    log(f"  near-ties {ties} of {cfg.T}, flipped {flipped}")
    assert ties <= max(2, cfg.T // 500)


@pytest.mark.parametrize("T,E,K,hot", [(1, 16, 4, 0), (63, 16, 4, 0), (64, 256, 8, 0),
                                       (65, 256, 8, 2), (1000, 256, 8, 8), (8192, 256, 8, 0),
                                       (16384, 256, 8, 8), (4096, 8, 8, 0), (100, 256, 1, 3)])
def test_permute_bit_exact(T, E, K, hot):
    log(f"permute T={T} E={E} K={K} hot={hot}")
    cfg = workloads.get("decode_bf16").replace(T=T, E=E, K=K, G=1, M=1, topn=1)
    idx = workloads.make_topk_indices(T, E, K, hot=hot, hot_weight=0.7)
    out = permute(cfg, idx.cuda())
    load, off, row_token, pair_row = oracle.permute(idx.numpy(), E)
    np.testing.assert_array_equal(out["load"].cpu().numpy(), load)
    np.testing.assert_array_equal(out["offsets"].cpu().numpy(), off)
    np.testing.assert_array_equal(out["row_token"].cpu().numpy(), row_token)
    np.testing.assert_array_equal(out["pair_row"].cpu().numpy(), pair_row)


@pytest.mark.parametrize("E,T,K,seed", [(256, 8192, 8, 0), (256, 16384, 8, 1), (16, 64, 4, 2),
                                        (256, 127, 8, 3), (1, 5, 1, 4)])
def test_bias_update_bit_exact(E, T, K, seed):
    log(f"bias_update E={E} T={T} K={K}")
    cfg = workloads.get("decode_bf16").replace(T=T, E=E, K=K, G=1, M=1, topn=1)
    load = workloads.make_loads(E, T, K, seed=seed)
    g = torch.Generator().manual_seed(seed)
    bias = (torch.rand(E, generator=g) - 0.5) * 0.02
    gamma = 1e-3
    ref = oracle.bias_update(load.numpy(), bias.numpy(), gamma, T, K)
    b = bias.cuda()
    moe.moe_bias_update(config_of(cfg), load.cuda(), gamma, b)
    torch.cuda.synchronize()
    got = b.cpu().numpy()
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("w", ["e4m3", "e4m3_pow2"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (7, 7168), (300, 2048), (64, 256)])
def test_act_quant_bit_exact(rows, cols, w):
    log(f"act_quant rows={rows} cols={cols} weights={w}")
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = torch.randn((rows, cols), generator=g) * torch.exp(torch.randn((rows, 1), generator=g) * 3)
    x[0, :128] = 0.0                                       # zero block -> scale 1
    if cols >= 256:
        x[0, 128] = 448.0 * 2 ** -20                        # tiny block (subnormal codes)
    x = x.to(torch.bfloat16)
    if w == "e4m3_pow2" and rows > 1:
        x[1, :128] = 448.0 * 2.0 ** -130                   # scale floor 2^-126
        x[1, 128 % cols] = -448.0 * 2.0 ** 3               # amax exactly 448 * 2^3
    cfg = workloads.get("prefill_fp8").replace(w=w)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    moe.moe_act_quant_e4m3(config_of(cfg), x.cuda(), rows, cols, q, s)
    torch.cuda.synchronize()
    quant = oracle.quantize_1x128_pow2 if w == "e4m3_pow2" else oracle.quantize_1x128
    rq, rs = quant(x.float().numpy())
    assert s.cpu().numpy().tobytes() == rs.tobytes()
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_route_is_deterministic():
    cfg = workloads.get("decode_bf16").replace(T=1024)
    d = _router_inputs(cfg)
    ws = workspace(config_of(cfg))
    a = route(cfg, d, ws)
    b = route(cfg, d, ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
