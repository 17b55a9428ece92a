"""GPU parity of the auxiliary-loss-free balancing loop on the skewed workload.

T=16384 tokens, 8 hot experts (router logit offset +2.0), 50 steps of forward +
bias update with gamma = 1e-3, a fresh seeded batch per step.  Every step: routing
bit-exact outside near-ties, loads and the bias update bit-exact (a near-tie flip
excuses only the experts whose load it moved), outputs on 512 sampled rows at the
first and last step.  The per-step max/mean load of the free-running GPU loop is
printed (the pages report hot experts at about 8x the mean early in training).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import (TOL, compare_routing, config_of, expert_getter, layer_forward, log,
                         rel_err, workspace)

pytestmark = pytest.mark.gpu


def _trajectory(cfg, steps, compare_out_steps):
    """Lock-step check: every step both sides start from the oracle's bias b_s (an
    oracle value handed to the GPU), so each step's routing, loads and bias update
    are compared exactly and a near-tie flip cannot propagate.  Alongside, the GPU
    runs free with its own bias; its max/mean load trajectory is returned."""
    d = workloads.make_layer_inputs(cfg, device="cuda", step=0)
    c = config_of(cfg)
    ws = workspace(c)
    bias_free = d["bias"].clone()                       # free-running GPU trajectory
    bias_ora = d["bias"].cpu().numpy().astype(np.float32)
    get = expert_getter(cfg, d)
    mean = cfg.T * cfg.K / cfg.E
    ratios, flip_steps = [], []
    for s in range(steps):
        if s > 0:
            d["x"] = workloads.make_tokens(cfg, step=s, device="cuda")
        # lock-step: GPU routed with the oracle's bias
        b_in = torch.from_numpy(bias_ora.copy()).cuda()
        out = layer_forward(cfg, dict(d, bias=b_in), ws=ws)
        r = oracle.route(d["x"], d["w_router"], bias_ora, cfg.G, cfg.M, cfg.topn, cfg.K)
        load_ora, *_ = oracle.permute(r.idx, cfg.E)
        load_gpu = out["load"].cpu().numpy()
        ties = compare_routing(r, out["idx"], out["gate"], where=f"step {s}")
        same_load = load_gpu == load_ora
        if not same_load.all():
            gi = np.sort(out["idx"].cpu().numpy(), axis=1)
            flips = np.nonzero(np.any(gi != np.sort(r.idx, axis=1), axis=1))[0]
            assert len(flips) > 0 and np.all(r.near_tie[flips]), f"step {s}: loads differ outside near-ties"
            flip_steps.append((s, flips.tolist()))
            log(f"  step {s}: near-tie flips on tokens {flips.tolist()}")
        moe.moe_bias_update(c, out["load"], cfg.gamma, b_in)
        torch.cuda.synchronize()
        nb_ora = oracle.bias_update(load_ora, bias_ora, cfg.gamma, cfg.T, cfg.K)
        nb_gpu = b_in.cpu().numpy()
        assert nb_gpu[same_load].tobytes() == nb_ora[same_load].tobytes(), f"bias update differs at step {s}"
        if s in compare_out_steps:
            rows = workloads.sample_rows(cfg.T, 512, seed=s).numpy()
            same = np.all(out["idx"].cpu().numpy() == r.idx, axis=1)
            rows = rows[same[rows]]
            ref = oracle.layer_output(d["x"], r.idx, r.gate, get, cfg.E, cfg.Ns, rows=rows)
            err = rel_err(out["y"].float().cpu().numpy()[rows], ref)
            log(f"  step {s}: output rel err {err:.3e} on {len(rows)} rows")
            assert err <= TOL["bf16"]
        bias_ora = nb_ora
        # free-running GPU step (its own bias), for the load trajectory
        free = layer_forward(cfg, dict(d, bias=bias_free), ws=ws)
        moe.moe_bias_update(c, free["load"], cfg.gamma, bias_free)
        torch.cuda.synchronize()
        ratios.append(float(free["load"].max().item() / mean))
        log(f"  step {s:2d}: max/mean load {ratios[-1]:.3f} (oracle lock-step "
            f"{load_ora.max() / mean:.3f}), near-ties {ties}")
    return ratios, flip_steps


@pytest.mark.slow
def test_skewed_balancing_trajectory():
    cfg = workloads.get("skewed_bf16")
    log("skewed_bf16: T=16384, 8 hot experts, 50 steps, gamma=1e-3")
    ratios, flips = _trajectory(cfg, cfg.steps, compare_out_steps={0, cfg.steps - 1})
    log(f"  max/mean load: step 0 {ratios[0]:.2f}, step 10 {ratios[10]:.2f}, "
        f"step 49 {ratios[-1]:.2f}; near-tie flips {flips}")
    assert ratios[0] > 4.0                       # the hot experts are hot
    assert ratios[-1] < 0.5 * ratios[0]          # and the bias pulls them back


def test_balancing_small_checkpoint_resume():
    """25 + 25 steps with the bias saved and restored equals 50 straight steps."""
    cfg = workloads.get("skewed_bf16").replace(T=512, hidden=256, inter=256, E=16, K=4, G=4, M=2,
                                               gamma=2e-2)
    c = config_of(cfg)
    ws = workspace(c)
    d = workloads.make_layer_inputs(cfg, device="cuda")

    def run(bias, steps, start):
        for s in range(start, start + steps):
            d["x"] = workloads.make_tokens(cfg, step=s, device="cuda")
            out = layer_forward(cfg, dict(d, bias=bias), ws=ws)
            moe.moe_bias_update(c, out["load"], cfg.gamma, bias)
        torch.cuda.synchronize()
        return bias

    straight = run(d["bias"].clone(), 50, 0)
    half = run(d["bias"].clone(), 25, 0)
    saved = half.cpu().clone()                         # checkpoint: the only carried state
    resumed = run(saved.cuda(), 25, 25)
    assert torch.equal(straight, resumed)
