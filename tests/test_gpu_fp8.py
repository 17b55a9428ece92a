"""GPU parity of the FP8 paths (e4m3 weights with 128x128 block scales, activations
quantised per 1x128 on the fly; the block scales arbitrary fp32 values or powers of
two) against the float64 oracle.

Two references: the fp32 oracle (dequantised weights, unquantised activations: the
6e-2 bound of the FP8 workload) and the oracle's FP8-emulating expert (x and h
quantised per 1x128 exactly as the kernels do), which pins the kernel more tightly.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import (TOL, check_layer_stages, config_of, expert_getter, inputs_on_gpu,
                         layer_forward, log, oracle_route, rel_err, weights_of, workspace)

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=256, inter=256, E=16, K=4, G=4, M=2, topn=2)
# Against the fp32 oracle the FP8 method itself (the oracle's exact emulation of the
# quantisation, float64 sums) is off by 4.1e-2 .. 5.6e-2 on these shapes (global norm;
# most of it from quantising x).  Against the FP8-emulating oracle the remaining
# difference is the few e4m3 codes of h that flip because the kernel's h carries
# fp32-accumulation rounding before its bf16 rounding: one code step is 1/16 of the
# value, a handful per row out of `inter` terms gives a few 1e-3 (measured
# 3e-3..9e-3 on MI355X); bound 2e-2.
EMU_TOL = 2e-2
# the kernel's own share beyond the method's error when judged against the fp32 oracle
KERNEL_SHARE = 1e-2


def fp32_bound(method_err):
    """The workload's 6e-2 bar wherever the FP8 method itself leaves the kernel its
    1e-2 share (method error <= 5e-2); where the method alone takes more, the bar is
    the method's error plus that share (logged by the callers)."""
    return max(TOL["e4m3"], method_err + KERNEL_SHARE)


def _check(cfg, d, out, rows=None):
    r = oracle_route(cfg, d)
    idx_ref, gate_ref, _, flipped = check_layer_stages(cfg, r, out, where=cfg.name)
    rows = np.arange(cfg.T) if rows is None else np.asarray(rows)
    get = expert_getter(cfg, d)
    got = out["y"].float().cpu().numpy()[rows]
    ref = oracle.layer_output(d["x"], idx_ref, gate_ref, get, cfg.E, cfg.Ns, rows=rows)
    err = rel_err(got, ref)
    emu_ffn = (oracle.expert_ffn_fp8_pow2_emulated if cfg.w == "e4m3_pow2"
               else oracle.expert_ffn_fp8_emulated)
    emu = oracle.layer_output(d["x"], idx_ref, gate_ref, get, cfg.E, cfg.Ns, rows=rows, ffn=emu_ffn)
    err_emu = rel_err(got, emu)
    method = rel_err(emu, ref)
    log(f"  {cfg.name} ({cfg.w}): rows {len(rows)}, near-ties {int(r.near_tie.sum())}, flipped "
        f"{flipped}, rel err vs fp32 {err:.3e} (the FP8 method itself {method:.3e}, bar "
        f"{fp32_bound(method):.3e}), vs fp8-emulating {err_emu:.3e}")
    assert err <= fp32_bound(method), err
    assert err_emu <= EMU_TOL, err_emu


@pytest.mark.parametrize("over", [dict(T=37), dict(T=1), dict(T=300, seed=1), dict(T=64, Ns=0),
                                  dict(T=129, Ns=2, bias="uniform", bias_range=0.02),
                                  dict(T=200, E=64, G=8, M=4, K=6, inter=384, hidden=384)])
@pytest.mark.parametrize("w", ["e4m3", "e4m3_pow2"])
def test_layer_small_fp8(over, w):
    cfg = workloads.get("prefill_fp8").replace(**{**SMALL, **over, "w": w})
    log(f"layer small fp8 {w} {over}")
    d = inputs_on_gpu(cfg)
    _check(cfg, d, layer_forward(cfg, d))


@pytest.mark.parametrize("w", ["e4m3", "e4m3_pow2"])
def test_fp8_decode_shape(w):
    cfg = workloads.get("prefill_fp8").replace(T=128, bias="uniform", bias_range=0.01,
                                               compare_rows=None, w=w)
    log(f"layer fp8 decode shape (T=128, h=7168, E=256, {w})")
    d = inputs_on_gpu(cfg)
    out = layer_forward(cfg, d)
    _check(cfg, d, out)
    again = layer_forward(cfg, d)
    assert torch.equal(out["y"], again["y"]), "run-to-run difference"


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill_fp8", "prefill_fp8_pow2"])
def test_layer_prefill_fp8(name):
    cfg = workloads.get(name)
    log(f"layer {name} (T=8192): routing on all tokens, output on 512 sampled rows")
    d = inputs_on_gpu(cfg)
    out = layer_forward(cfg, d)
    _check(cfg, d, out, rows=workloads.sample_rows(cfg.T, cfg.compare_rows).numpy())
