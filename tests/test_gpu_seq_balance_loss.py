"""GPU parity of the router affinities and the sequence-wise balance loss.

moe_router_scores against the float64 affinities of the oracle, and bit-identical
to the affinities moe_route selected on (its gates are reproduced exactly from
them).  moe_balance_loss on seeded affinities and selections (both sides), and on
the GPU's own affinities with the oracle's selection against the oracle's own
affinities, logits and selection, to the float64 oracle's bar: f within one
rounding, P and the loss within 2e-5 relative, the logit gradient within 2e-5 of
its largest magnitude (fp32 sums of up to 8192 terms; the gradient's f_e minus
sum_i f_i s'_i cancels).  Sizes span one chunk, several chunks with a ragged last
chunk, one token per sequence, the batch-wise case and the prefill shape.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import config_of, log, workspace

pytestmark = pytest.mark.gpu

ALPHA = 1e-4


def _logit(s64):
    return np.log(s64 / (1.0 - s64))


def _run_loss(c, s, idx, L, alpha=ALPHA, ws=None, full=True):
    T, E = s.shape
    S = T // L
    ws = workspace(c) if ws is None else ws
    out = {"loss": torch.empty(S, dtype=torch.float32, device="cuda")}
    if full:
        out["f"] = torch.empty((S, E), dtype=torch.float32, device="cuda")
        out["P"] = torch.empty((S, E), dtype=torch.float32, device="cuda")
        out["grad"] = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_balance_loss(c, s, idx, L, alpha, out["loss"], out.get("f"), out.get("P"),
                         out.get("grad"), ws)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in out.items()}


def _oracle(s64, z64, idx, L, K, alpha=ALPHA):
    loss, f, P = oracle.balance_loss(s64, idx, L, alpha, K)
    return {"loss": loss, "f": f, "P": P,
            "grad": oracle.balance_loss_grad_logits(z64, idx, L, alpha, K)}


def _compare(got, want):
    np.testing.assert_allclose(got["f"], want["f"], rtol=1e-7, atol=0)
    np.testing.assert_allclose(got["P"], want["P"], rtol=2e-5, atol=0)
    np.testing.assert_allclose(got["loss"], want["loss"], rtol=2e-5, atol=0)
    gerr = np.abs(got["grad"] - want["grad"]).max() / np.abs(want["grad"]).max()
    log(f"  loss[0] {got['loss'][0]:.6e} (oracle {want['loss'][0]:.6e}); grad rel err {gerr:.2e}")
    assert gerr <= 2e-5


def _check_against_oracle(got, s_cpu, idx_cpu, L, K):
    """Both sides on the same seeded generator outputs (affinities, selections)."""
    s64 = s_cpu.double().numpy()
    _compare(got, _oracle(s64, _logit(s64), idx_cpu.numpy(), L, K))


def _cfg(T, E, K, G):
    # hidden/inter only size the workspace here
    return moe.make_config(T, 256, 128, E, K, G, G, 1, 0, "f32", "f32")


@pytest.mark.parametrize("T,E,K,L", [(64, 16, 4, 64), (64, 16, 4, 16), (64, 16, 4, 1),
                                     (300, 16, 4, 100), (130, 256, 8, 65), (96, 200, 6, 96),
                                     (8192, 256, 8, 4096), (8192, 256, 8, 8192)])
def test_balance_loss_matches_oracle(T, E, K, L):
    log(f"balance loss T={T} E={E} K={K} seq_len={L}")
    s = workloads.make_affinities(T, E, seed=T + E)
    idx = workloads.make_topk_indices(T, E, K, seed=T + K)
    c = _cfg(T, E, K, 4 if E % 4 == 0 else 1)
    got = _run_loss(c, s.cuda(), idx.cuda(), L)
    _check_against_oracle(got, s, idx, L, K)


def test_balance_loss_optional_outputs_and_determinism():
    T, E, K, L = 8192, 256, 8, 4096
    log("balance loss optional outputs / determinism")
    s = workloads.make_affinities(T, E, seed=1).cuda()
    idx = workloads.make_topk_indices(T, E, K, seed=1).cuda()
    c = _cfg(T, E, K, 8)
    ws = workspace(c)
    a = _run_loss(c, s, idx, L, ws=ws)
    b = _run_loss(c, s, idx, L, ws=ws)
    only = _run_loss(c, s, idx, L, ws=ws, full=False)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_array_equal(only["loss"], a["loss"])
    # the gradient without a caller f buffer (f kept in the workspace) is the same
    grad = torch.empty((T, E), dtype=torch.float32, device="cuda")
    loss = torch.empty(T // L, dtype=torch.float32, device="cuda")
    moe.moe_balance_loss(c, s, idx, L, ALPHA, loss, None, None, grad, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(grad.cpu().double().numpy(), a["grad"])


def test_balance_loss_closed_forms_on_gpu():
    # perfectly balanced selection -> f = 1, loss = alpha whatever the affinities;
    # full concentration with the affinity mass on the chosen experts -> alpha E / K
    T, E, K, L = 128, 16, 4, 32
    c = _cfg(T, E, K, 4)
    s = workloads.make_affinities(T, E, seed=7)
    idx = torch.tensor([[(K * t + k) % E for k in range(K)] for t in range(T)], dtype=torch.int32)
    got = _run_loss(c, s.cuda(), idx.cuda(), L)
    np.testing.assert_array_equal(got["f"], 1.0)
    np.testing.assert_allclose(got["loss"], ALPHA, rtol=2e-6)
    assert np.abs(got["grad"]).max() <= 1e-6 * ALPHA
    s2 = torch.full((T, E), 1e-30, dtype=torch.float32)
    s2[:, :K] = 0.5
    idx2 = torch.arange(K, dtype=torch.int32).repeat(T, 1)
    got2 = _run_loss(c, s2.cuda(), idx2.cuda(), L)
    np.testing.assert_allclose(got2["loss"], ALPHA * E / K, rtol=2e-6)


def test_out_of_range_selections_are_not_counted():
    T, E, K, L = 64, 16, 4, 32
    c = _cfg(T, E, K, 4)
    s = workloads.make_affinities(T, E, seed=3)
    idx = workloads.make_topk_indices(T, E, K, seed=3)
    bad = idx.clone()
    bad[::5, 1] = E + 3
    bad[::7, 2] = -1
    got = _run_loss(c, s.cuda(), bad.cuda(), L)
    good = bad.numpy()
    for q in range(T // L):
        sel = good[q * L:(q + 1) * L].ravel()
        sel = sel[(sel >= 0) & (sel < E)]
        expect = E / (K * L) * np.bincount(sel, minlength=E)
        np.testing.assert_allclose(got["f"][q], expect, rtol=1e-7, atol=0)


@pytest.mark.parametrize("name", ["tiny_fp32", "decode_bf16", "prefill_bf16"])
def test_router_scores_and_loss_on_the_router_outputs(name):
    """moe_router_scores against the oracle's affinities; then the loss of the whole
    chain: the GPU on its own affinities with the oracle's selection (an oracle value
    handed to the GPU), the oracle on its own affinities, logits and selection."""
    cfg = workloads.get(name)
    log(f"router scores + balance loss on {name}")
    c = config_of(cfg)
    x = workloads.make_tokens(cfg)
    w_r = workloads.make_router(cfg)
    bias = workloads.make_bias(cfg)
    ws = workspace(c)
    scores = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    gate = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    moe.moe_router_scores(c, x.cuda(), w_r.cuda(), scores, ws)
    moe.moe_route(c, x.cuda(), w_r.cuda(), bias.cuda(), idx, gate, ws)
    torch.cuda.synchronize()
    s = scores.cpu()
    z64, s64 = oracle.affinities(x, w_r)
    err = np.abs(s.double().numpy() - s64).max()
    log(f"  max |s - oracle| = {err:.2e}")
    assert err <= (1e-6 if cfg.act == "f32" else 1e-5)
    # property: the gates of moe_route are these very affinities normalised in k order
    sel = torch.gather(s, 1, idx.cpu().long())
    total = sel[:, 0].clone()
    for k in range(1, cfg.K):
        total = total + sel[:, k]
    assert torch.equal(gate.cpu(), sel / total[:, None])
    r = oracle.route(x, w_r, bias.numpy(), cfg.G, cfg.M, cfg.topn, cfg.K)
    L = cfg.T // 2
    got = _run_loss(c, scores, torch.from_numpy(r.idx).cuda(), L, ws=ws)
    _compare(got, _oracle(s64, z64, r.idx, L, cfg.K))
