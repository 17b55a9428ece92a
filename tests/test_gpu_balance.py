"""GPU parity of the auxiliary-loss-free balancing loop on the skewed workload.

T=16384 tokens, 8 hot experts (router logit offset +2.0), 50 steps of forward +
bias update with gamma = 1e-3, a fresh seeded batch per step.  Every step: routing
bit-exact outside near-ties (a valid alternative of the oracle's at near-ties), the
loads of every expert and the bias update of every expert bit-exact against the
oracle's permutation and update of the reference selection, outputs on 512 sampled
rows at the first and last step.  Beside it the GPU and the oracle each run the loop
free (each carrying its own bias); their max/mean load trajectories and the point
where their biases part (only after a near-tie flip) are reported (the pages report
hot experts at about 8x the mean early in training).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import (TOL, check_layer_stages, check_routing, config_of, expert_getter,
                         layer_forward, log, rel_err, workspace)

pytestmark = pytest.mark.gpu


def _trajectory(cfg, steps, compare_out_steps):
    """Lock-step check: every step both sides start from the oracle's bias b_s (an
    oracle value handed to the GPU), so each step's routing, loads and bias update
    are compared exactly and a near-tie flip cannot propagate.  Alongside, the GPU
    and the oracle each run free with their own bias; while the two free biases are
    equal bit for bit, the free GPU step is judged like the lock-step one and the
    biases must stay equal unless a near-tie token flipped."""
    d = workloads.make_layer_inputs(cfg, device="cuda", step=0)
    c = config_of(cfg)
    ws = workspace(c)
    bias_free = d["bias"].clone()                       # free-running GPU trajectory
    bias_ora = d["bias"].cpu().numpy().astype(np.float32)
    bias_free_ora = bias_ora.copy()                     # free-running oracle trajectory
    get = expert_getter(cfg, d)
    mean = cfg.T * cfg.K / cfg.E
    traj = {"gpu_free": [], "oracle_free": [], "lock_step": []}
    flip_steps, parted = [], None
    for s in range(steps):
        if s > 0:
            d["x"] = workloads.make_tokens(cfg, step=s, device="cuda")
        _, aff = oracle.affinities(d["x"], d["w_router"])
        # lock-step: GPU routed with the oracle's bias
        b_in = torch.from_numpy(bias_ora.copy()).cuda()
        out = layer_forward(cfg, dict(d, bias=b_in), ws=ws)
        r = oracle.select(aff, bias_ora, cfg.G, cfg.M, cfg.topn, cfg.K)
        idx_ref, gate_ref, load_ref, flipped = check_layer_stages(cfg, r, out, where=f"step {s}")
        if flipped:
            flip_steps.append((s, flipped))
        moe.moe_bias_update(c, out["load"], cfg.gamma, b_in)
        torch.cuda.synchronize()
        nb_ora = oracle.bias_update(load_ref, bias_ora, cfg.gamma, cfg.T, cfg.K)
        assert b_in.cpu().numpy().tobytes() == nb_ora.tobytes(), f"bias update differs at step {s}"
        if s in compare_out_steps:
            rows = workloads.sample_rows(cfg.T, 512, seed=s).numpy()
            ref = oracle.layer_output(d["x"], idx_ref, gate_ref, get, cfg.E, cfg.Ns, rows=rows)
            err = rel_err(out["y"].float().cpu().numpy()[rows], ref)
            log(f"  step {s}: output rel err {err:.3e} on {len(rows)} rows")
            assert err <= TOL["bf16"]
        bias_ora = nb_ora
        # the free-running loops: the GPU with its own bias, the oracle with its own
        same_start = bias_free.cpu().numpy().tobytes() == bias_free_ora.tobytes()
        free = layer_forward(cfg, dict(d, bias=bias_free), ws=ws)
        moe.moe_bias_update(c, free["load"], cfg.gamma, bias_free)
        rf = oracle.select(aff, bias_free_ora, cfg.G, cfg.M, cfg.topn, cfg.K)
        load_free_ora, *_ = oracle.permute(rf.idx, cfg.E)
        bias_free_ora = oracle.bias_update(load_free_ora, bias_free_ora, cfg.gamma, cfg.T, cfg.K)
        torch.cuda.synchronize()
        bf_gpu = bias_free.cpu().numpy()
        if same_start:
            _, _, fflip = check_routing(cfg, rf, free["idx"], free["gate"], where=f"free step {s}")
            if not fflip:
                np.testing.assert_array_equal(free["load"].cpu().numpy(), load_free_ora)
                assert bf_gpu.tobytes() == bias_free_ora.tobytes(), f"free loops part at step {s}"
            elif bf_gpu.tobytes() != bias_free_ora.tobytes():
                parted = (s, fflip)
        nd = int(np.sum(bf_gpu != bias_free_ora))
        traj["gpu_free"].append(float(free["load"].max().item() / mean))
        traj["oracle_free"].append(float(load_free_ora.max() / mean))
        traj["lock_step"].append(float(load_ref.max() / mean))
        log(f"  step {s:2d}: max/mean load GPU free {traj['gpu_free'][-1]:.3f}, oracle free "
            f"{traj['oracle_free'][-1]:.3f}, lock-step {traj['lock_step'][-1]:.3f}; near-ties "
            f"{int(r.near_tie.sum())}, flipped {flipped}; free biases differ on {nd} experts "
            f"(max {np.abs(bf_gpu - bias_free_ora).max() / cfg.gamma:.0f} gamma)")
    return traj, flip_steps, parted


@pytest.mark.slow
def test_skewed_balancing_trajectory():
    cfg = workloads.get("skewed_bf16")
    log("skewed_bf16: T=16384, 8 hot experts, 50 steps, gamma=1e-3")
    traj, flips, parted = _trajectory(cfg, cfg.steps, compare_out_steps={0, cfg.steps - 1})
    g = traj["gpu_free"]
    log(f"  max/mean load (GPU free): step 0 {g[0]:.2f}, step 10 {g[10]:.2f}, step 49 {g[-1]:.2f}; "
        f"oracle free: {traj['oracle_free'][0]:.2f}, {traj['oracle_free'][10]:.2f}, "
        f"{traj['oracle_free'][-1]:.2f}; lock-step near-tie flips {flips}; free loops part at "
        f"{parted if parted else 'no step'}")
    assert g[0] > 4.0                            # the hot experts are hot
    assert g[-1] < 0.5 * g[0]                    # and the bias pulls them back
    assert traj["oracle_free"][-1] < 0.5 * traj["oracle_free"][0]


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
