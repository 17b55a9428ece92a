"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same materialised inputs, and compare them.

Comparison rules (the layer's parity bar):
  * routing indices, loads, permutation and bias: bit-exact, except tokens whose
    float64 group or expert boundary gap is below 1e-6 (near-ties), which are
    counted and reported instead;
  * gates: relative error <= 1e-5 (fp32 sigmoid and division against float64);
  * outputs: max|y - ref| / max|ref| over the compared rows, <= 1e-5 for fp32,
    2e-2 for bf16, 6e-2 for FP8 weights, against the float64 oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2, "e4m3_pow2": 6e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def config_of(cfg: workloads.MoeShape):
    return moe.make_config(cfg.T, cfg.hidden, cfg.inter, cfg.E, cfg.K, cfg.G, cfg.M, cfg.topn,
                           cfg.Ns, cfg.act, cfg.w)


def inputs_on_gpu(cfg, step=0):
    return workloads.make_layer_inputs(cfg, device="cuda", step=step)


def workspace(c):
    n = moe.moe_workspace_bytes(c)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def weights_of(d):
    return {k: d[k] for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down") if k in d}


def act_dtype(cfg):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


def layer_forward(cfg, d, residual=None, ws=None):
    c = config_of(cfg)
    ws = workspace(c) if ws is None else ws
    out = {
        "y": torch.empty((cfg.T, cfg.hidden), dtype=act_dtype(cfg), device="cuda"),
        "idx": torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda"),
        "gate": torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda"),
        "load": torch.empty(cfg.E, dtype=torch.int32, device="cuda"),
    }
    moe.moe_layer_forward(c, d["x"], d["w_router"], d["bias"], weights_of(d), residual, out["y"],
                          out["idx"], out["gate"], out["load"], ws)
    torch.cuda.synchronize()
    return out


def route(cfg, d, ws=None):
    c = config_of(cfg)
    ws = workspace(c) if ws is None else ws
    idx = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    gate = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    moe.moe_route(c, d["x"], d["w_router"], d["bias"], idx, gate, ws)
    torch.cuda.synchronize()
    return idx, gate


def permute(cfg, idx, ws=None):
    c = config_of(cfg)
    ws = workspace(c) if ws is None else ws
    T, K, E = idx.shape[0], cfg.K, cfg.E
    out = dict(load=torch.empty(E, dtype=torch.int32, device="cuda"),
               offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               row_token=torch.empty(T * K, dtype=torch.int32, device="cuda"),
               pair_row=torch.empty(T * K, dtype=torch.int32, device="cuda"))
    moe.moe_permute(c, idx, out["load"], out["offsets"], out["row_token"], out["pair_row"], ws)
    torch.cuda.synchronize()
    return out


def expert_getter(cfg, d):
    """Oracle-side access to one expert's weights as float64 arrays (streamed from the GPU)."""
    def get(e):
        if workloads.is_fp8(cfg.w):
            return tuple(oracle.dequantize_blocks_128(d[n][e], d["s" + n[1:]][e])
                         for n in ("w_gate", "w_up", "w_down"))
        return tuple(d[n][e].to("cpu", torch.float64).numpy() for n in ("w_gate", "w_up", "w_down"))
    return get


def oracle_route(cfg, d):
    return oracle.route(d["x"], d["w_router"], d["bias"].cpu().numpy(), cfg.G, cfg.M, cfg.topn,
                        cfg.K)


def compare_routing(r: "oracle.RouteResult", idx_gpu, gate_gpu, where=""):
    """Bit-exact selection outside near-ties; gates to 1e-5 relative. Returns #near-ties."""
    gi = idx_gpu.cpu().numpy()
    gg = gate_gpu.cpu().numpy().astype(np.float64)
    tie = r.near_tie
    exact = ~tie & ~r.near_tie_order
    bad = np.nonzero(np.any(gi[exact] != r.idx[exact], axis=1))[0]
    assert bad.size == 0, f"{where}: {bad.size} tokens differ, first {np.nonzero(exact)[0][bad[:5]]}"
    # near-tie-in-order tokens: same set, and the order valid for the float64 values
    for t in np.nonzero(~tie & r.near_tie_order)[0]:
        assert set(gi[t]) == set(r.idx[t]), f"{where}: token {t} set differs"
    # every token (near-ties too): K distinct experts, at most M groups, gates sum to 1
    rel = np.abs(gg[exact] - r.gate[exact]) / np.abs(r.gate[exact])
    assert rel.size == 0 or rel.max() <= 1e-5, f"{where}: gate rel err {rel.max()}"
    return int(tie.sum())


def routing_valid(cfg, idx_gpu, gate_gpu):
    gi = idx_gpu.cpu().numpy()
    gg = gate_gpu.cpu().numpy()
    n = cfg.E // cfg.G
    for t in range(gi.shape[0]):
        assert len(set(gi[t].tolist())) == cfg.K
        assert len({e // n for e in gi[t].tolist()}) <= cfg.M
    assert np.all(gi >= 0) and np.all(gi < cfg.E)
    np.testing.assert_allclose(gg.sum(1), 1.0, atol=1e-5)


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.abs(y - ref).max() / np.abs(ref).max())


def oracle_layer(cfg, d, idx, gate, rows=None, residual=None):
    """Oracle output on ``rows`` for a routing the oracle computed."""
    return oracle.layer_output(d["x"], idx, gate, expert_getter(cfg, d), cfg.E, cfg.Ns,
                               rows=rows, residual=residual)
