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


def check_routing(cfg, r: "oracle.RouteResult", idx_gpu, gate_gpu, where=""):
    """Judge the GPU's selection and gates against the oracle and return the oracle's
    reference for them: (idx_ref [T, K], gate_ref [T, K] float64, flipped tokens).

    * tokens without near-ties: indices bit-exact (order included), gates to 1e-5;
    * tokens with two selected experts within 1e-6 (order-only near-ties): the same
      set, and the GPU's order non-increasing in the float64 biased affinity within
      1e-6;
    * tokens whose group or expert boundary gap is below 1e-6: the GPU's set must be
      one of the selections the oracle enumerates as valid (oracle.valid_selections:
      a top-M group set and a top-K of it, both within 1e-6), in a valid order;
    * every token: K distinct experts in range, at most M groups, gates equal to
      s / sum(s) over the selection (float64 oracle affinities) within 1e-5.
    Where several selections are valid, the reference row is the oracle's alternative
    that the GPU chose, in the GPU's (validated) order, with the oracle's float64
    gates for it: every value in idx_ref / gate_ref is an oracle value."""
    gi = idx_gpu.cpu().numpy().astype(np.int64)
    gg = gate_gpu.cpu().numpy().astype(np.float64)
    T, K = gi.shape
    E, G, M = cfg.E, cfg.G, cfg.M
    assert np.all((gi >= 0) & (gi < E)), f"{where}: expert index out of range"
    srt = np.sort(gi, axis=1)
    assert K == 1 or np.all(np.diff(srt, axis=1) > 0), f"{where}: repeated expert"
    grp = np.sort(gi // (E // G), axis=1)
    ngroups = 1 + (np.diff(grp, axis=1) > 0).sum(1) if K > 1 else np.ones(T, int)
    assert np.all(ngroups <= M), f"{where}: more than M groups"
    tie = r.near_tie
    exact = ~tie & ~r.near_tie_order
    bad = np.nonzero(np.any(gi[exact] != r.idx[exact], axis=1))[0]
    assert bad.size == 0, f"{where}: {bad.size} tokens differ, first {np.nonzero(exact)[0][bad[:5]]}"
    idx_ref = r.idx.astype(np.int64).copy()
    flipped = []
    for t in np.nonzero(~exact)[0]:
        gset = frozenset(gi[t].tolist())
        if tie[t]:
            ok = gset in oracle.valid_selections(r.sb[t], G, M, cfg.topn, K)
            assert ok, f"{where}: token {t} selection {sorted(gset)} is not valid"
        else:
            assert gset == frozenset(r.idx[t].tolist()), f"{where}: token {t} set differs"
        sbt = r.sb[t, gi[t]]
        assert np.all(np.diff(sbt) <= 1e-6), f"{where}: token {t} order invalid"
        idx_ref[t] = gi[t]                       # the oracle's alternative, GPU order
        if gset != frozenset(r.idx[t].tolist()):
            flipped.append(int(t))
    ss = np.take_along_axis(r.s, idx_ref, 1)
    gate_ref = ss / ss.sum(1, keepdims=True)
    rel = np.abs(gg - gate_ref) / gate_ref
    assert rel.max() <= 1e-5, f"{where}: gate rel err {rel.max()}"
    return idx_ref.astype(np.int32), gate_ref, flipped


def check_layer_stages(cfg, r, out, where=""):
    """Routing (check_routing), then the loads of every expert bit-exact against the
    oracle's permutation of the reference selection.  Returns (idx_ref, gate_ref,
    load_ref, flipped)."""
    idx_ref, gate_ref, flipped = check_routing(cfg, r, out["idx"], out["gate"], where)
    load_ref, *_ = oracle.permute(idx_ref, cfg.E)
    np.testing.assert_array_equal(out["load"].cpu().numpy(), load_ref, err_msg=f"{where}: loads")
    return idx_ref, gate_ref, load_ref, flipped


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.abs(y - ref).max() / np.abs(ref).max())


def oracle_layer(cfg, d, idx, gate, rows=None, residual=None):
    """Oracle output on ``rows`` for a routing the oracle computed."""
    return oracle.layer_output(d["x"], idx, gate, expert_getter(cfg, d), cfg.E, cfg.Ns,
                               rows=rows, residual=residual)
