"""GPU parity of the grouped FFN, the combine and the whole layer forward.

The layer's routing is judged token by token (bit-exact outside near-ties, a valid
alternative of the oracle's at near-ties), its loads on every expert, and its output
on every compared row against the oracle run on the reference selection (a flipped
near-tie token is compared on the oracle's alternative it chose).  The grouped FFN
and the combine are also driven directly with the oracle's own routing and
permutation so they are checked stage by stage.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import (TOL, act_dtype, check_layer_stages, config_of, expert_getter,
                         inputs_on_gpu, layer_forward, log, oracle_layer, oracle_route, rel_err,
                         weights_of, workspace)

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=256, inter=256, E=16, K=4, G=4, M=2, topn=2)


def _check_layer(cfg, d, out, rows=None, residual=None):
    r = oracle_route(cfg, d)
    idx_ref, gate_ref, _, flipped = check_layer_stages(cfg, r, out, where=cfg.name)
    rows = np.arange(cfg.T) if rows is None else np.asarray(rows)
    ref = oracle_layer(cfg, d, idx_ref, gate_ref, rows=rows, residual=residual)
    got = out["y"].float().cpu().numpy()[rows]
    err = rel_err(got, ref)
    log(f"  {cfg.name}: rows {len(rows)}, near-ties {int(r.near_tie.sum())}, flipped {flipped}, "
        f"rel err {err:.3e}")
    assert err <= TOL[cfg.w], err
    fl = np.intersect1d(rows, flipped)
    if fl.size:                                       # the flipped rows on their own
        sub = np.searchsorted(rows, fl)
        assert rel_err(got[sub], ref[sub]) <= TOL[cfg.w]
    return err


@pytest.mark.parametrize("over", [{}, dict(T=1), dict(T=5, K=1, M=1), dict(Ns=0), dict(Ns=2),
                                  dict(T=130, bias="uniform", bias_range=0.05)])
def test_layer_tiny_fp32(over):
    cfg = workloads.get("tiny_fp32").replace(**over)
    log(f"layer tiny_fp32 {over}")
    d = inputs_on_gpu(cfg)
    _check_layer(cfg, d, layer_forward(cfg, d))


@pytest.mark.parametrize("over", [dict(T=37), dict(T=1), dict(T=300, seed=1), dict(T=64, Ns=0),
                                  dict(T=129, Ns=2, bias="uniform", bias_range=0.02),
                                  dict(T=500, E=64, G=8, M=4, K=6, inter=384)])
def test_layer_small_bf16(over):
    cfg = workloads.get("decode_bf16").replace(**{**SMALL, **over})
    log(f"layer small bf16 {over}")
    d = inputs_on_gpu(cfg)
    _check_layer(cfg, d, layer_forward(cfg, d))


def test_layer_residual_bf16():
    cfg = workloads.get("decode_bf16").replace(T=50, **SMALL)
    d = inputs_on_gpu(cfg)
    out = layer_forward(cfg, d, residual=d["x"])
    _check_layer(cfg, d, out, residual=d["x"])


def test_grouped_ffn_and_combine_stagewise():
    """moe_grouped_ffn and moe_combine fed with the oracle's routing and permutation."""
    cfg = workloads.get("decode_bf16").replace(T=96, **SMALL)
    d = inputs_on_gpu(cfg)
    r = oracle_route(cfg, d)
    load, off, row_token, pair_row = oracle.permute(r.idx, cfg.E)
    c = config_of(cfg)
    ws = workspace(c)
    y_rows = torch.empty((cfg.rows, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    moe.moe_grouped_ffn(c, d["x"], cu(off), cu(row_token), weights_of(d), y_rows, ws)
    gate = cu(r.gate.astype(np.float32))
    y = torch.empty((cfg.T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(c, y_rows, cu(pair_row), gate, None, y)
    torch.cuda.synchronize()
    get = expert_getter(cfg, d)
    x64 = d["x"].double().cpu().numpy()
    yr = y_rows.float().cpu().numpy()
    for e in range(cfg.E):
        if load[e]:
            toks = row_token[off[e]:off[e + 1]]
            ref = oracle.expert_ffn(x64[toks], *get(e))
            assert rel_err(yr[off[e]:off[e + 1]], ref) <= TOL["bf16"], e
    ref_shared = oracle.expert_ffn(x64, *get(cfg.E))
    assert rel_err(yr[cfg.T * cfg.K:], ref_shared) <= TOL["bf16"]
    ref = oracle.layer_output(d["x"], r.idx, r.gate.astype(np.float32), get, cfg.E, cfg.Ns)
    assert rel_err(y.float().cpu().numpy(), ref) <= TOL["bf16"]


def test_layer_decode_bf16():
    cfg = workloads.get("decode_bf16")
    log("layer decode_bf16 (T=128, h=7168, E=256)")
    d = inputs_on_gpu(cfg)
    out = layer_forward(cfg, d)
    _check_layer(cfg, d, out)
    again = layer_forward(cfg, d)
    for k in out:
        assert torch.equal(out[k], again[k]), f"run-to-run difference in {k}"


@pytest.mark.slow
def test_layer_prefill_bf16():
    cfg = workloads.get("prefill_bf16")
    log("layer prefill_bf16 (T=8192): routing on all tokens, output on 512 sampled rows")
    d = inputs_on_gpu(cfg)
    out = layer_forward(cfg, d)
    _check_layer(cfg, d, out, rows=workloads.sample_rows(cfg.T, cfg.compare_rows).numpy())


@pytest.mark.slow
def test_layer_largest_batch_bf16():
    """The largest batch the 32-bit buffer offsets allow at the prefill shape (T = 58225,
    524025 grouped rows): routing on all tokens, output on sampled rows plus the last
    tokens (the ragged end of the token range and of the shared expert's rows)."""
    T = 58225
    cfg = workloads.get("prefill_bf16").replace(T=T)
    log(f"layer bf16 at the largest batch T={T}")
    d = inputs_on_gpu(cfg)
    out = layer_forward(cfg, d)
    rows = np.union1d(workloads.sample_rows(T, 96, seed=3).numpy(), np.arange(T - 8, T))
    _check_layer(cfg, d, out, rows=rows)

