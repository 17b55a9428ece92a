"""GPU parity of the combine and gate backward against the float64 oracle.

Inputs come from the seeded generators (output gradients, expert rows, gates,
affinities, selections) and the oracle (the permutation).  Bar: dgate within 2e-6 of
its largest magnitude (fp32 sums over hidden: exact bf16 products, about 30 terms
per thread, then fixed trees); the routed row gradients within one rounding of the
exact product (2^-8 relative for bf16, 2^-23 for fp32); the shared rows exact copies
of dy; the logit gradient within 5e-6 of its largest magnitude (a few fp32 roundings),
exactly zero (or exactly the accumulated base) on the experts not selected.  At
T = 8192 the combine is compared on a seeded subset of tokens, the oracle run on
the subset's own rows.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import log

pytestmark = pytest.mark.gpu


def _cfg(T, H, E, K, Ns, act):
    G = 4 if E % 4 == 0 else 1
    return moe.make_config(T, H, 128, E, K, G, G, 1, Ns, act, act)


@pytest.mark.parametrize("T,H,E,K,Ns,act", [(64, 256, 16, 4, 1, "f32"), (37, 256, 16, 4, 2, "bf16"),
                                            (5, 128, 8, 1, 0, "bf16"), (130, 7168, 256, 8, 1, "bf16"),
                                            (8192, 7168, 256, 8, 1, "bf16")])
def test_combine_backward(T, H, E, K, Ns, act):
    log(f"combine backward T={T} h={H} E={E} K={K} Ns={Ns} {act}")
    idx = workloads.make_topk_indices(T, E, K, seed=T)
    _, _, _, pair_row = oracle.permute(idx.numpy(), E)
    rows = T * K + T * Ns
    dy = workloads.make_dense((T, H), act, seed=T, name="dy")
    Y = workloads.make_dense((rows, H), act, seed=T, name="y_rows")
    g = workloads.make_gates(T, K, seed=T)
    dt = dy.dtype
    dgate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dY = torch.empty((rows, H), dtype=dt, device="cuda")
    moe.moe_combine_backward(_cfg(T, H, E, K, Ns, act), dy.cuda(), Y.cuda(),
                             torch.from_numpy(pair_row.astype(np.int32)).cuda(), g.cuda(), dgate, dY)
    torch.cuda.synchronize()
    toks = workloads.sample_rows(T, 256, seed=1).numpy()
    n = len(toks)
    # the oracle on the chosen tokens' own rows: routed pairs first, then shared rows
    routed = pair_row.reshape(T, K)[toks].ravel()
    shared = np.concatenate([T * K + s * T + toks for s in range(Ns)]) if Ns else np.zeros(0, int)
    sub_rows = np.concatenate([routed, shared]).astype(np.int64)
    want_dg, want_dY = oracle.combine_backward(dy[toks], Y[sub_rows], np.arange(n * K), g[toks],
                                               n, K, Ns)
    got_dg = dgate.cpu().double().numpy()[toks]
    err = np.abs(got_dg - want_dg).max() / np.abs(want_dg).max()
    got_dY = dY.cpu()[sub_rows].double().numpy()
    rel = 2.0 ** -8 if act == "bf16" else 2.0 ** -23
    row_err = np.abs(got_dY[:n * K] - want_dY[:n * K]) - rel * np.abs(want_dY[:n * K])
    log(f"  dgate rel err {err:.2e}; routed row excess over one rounding {row_err.max():.2e}")
    assert err <= 2e-6
    assert np.all(row_err <= 0)
    if Ns:
        np.testing.assert_array_equal(got_dY[n * K:], want_dY[n * K:])      # exact copies


@pytest.mark.parametrize("T,E,K", [(64, 16, 4), (130, 256, 8), (8192, 256, 8), (96, 200, 6),
                                   (5, 8, 1)])
def test_gate_backward(T, E, K):
    log(f"gate backward T={T} E={E} K={K}")
    s = workloads.make_affinities(T, E, seed=T + 1)
    idx = workloads.make_topk_indices(T, E, K, seed=T + 1)
    dg = workloads.make_dense((T, K), "f32", seed=T + 1, name="dgate")
    c = _cfg(T, 256, E, K, 1, "f32")
    s64 = s.double().numpy()
    want = oracle.gate_backward(np.log(s64 / (1 - s64)), idx.numpy(), dg)
    grad = torch.full((T, E), 7.0, dtype=torch.float32, device="cuda")    # overwritten
    moe.moe_gate_backward(c, s.cuda(), idx.cuda(), dg.cuda(), grad, accumulate=False)
    base = workloads.make_dense((T, E), "f32", seed=T + 2, name="base")
    acc = base.cuda()
    moe.moe_gate_backward(c, s.cuda(), idx.cuda(), dg.cuda(), acc, accumulate=True)
    torch.cuda.synchronize()
    got = grad.cpu().double().numpy()
    mask = np.ones((T, E), bool)
    np.put_along_axis(mask, idx.long().numpy(), False, axis=1)
    assert np.all(got[mask] == 0.0)
    np.testing.assert_array_equal(acc.cpu().numpy()[mask], base.numpy()[mask])
    if K == 1:                              # a single gate is always 1: no gradient
        assert np.all(got == 0.0)
        return
    scale = np.abs(want).max()
    err = np.abs(got - want).max() / scale
    err_acc = np.abs(acc.cpu().double().numpy() - (base.double().numpy() + want)).max() / scale
    log(f"  grad rel err {err:.2e}, accumulated {err_acc:.2e}")
    assert err <= 5e-6 and err_acc <= 5e-6


@pytest.mark.parametrize("rows,inter,act", [(1, 128, "bf16"), (37, 256, "bf16"), (300, 2048, "bf16"),
                                            (64, 128, "f32"), (65536, 2048, "bf16")])
def test_swiglu_backward(rows, inter, act):
    """Elementwise: each output within one rounding of the exact value plus 1e-5 of the
    array's largest magnitude (fp32 cancellation in silu' near its zero at a = -1.28);
    the 65536-row case on sampled rows."""
    log(f"swiglu backward rows={rows} inter={inter} {act}")
    a = workloads.make_dense((rows, inter), act, std=2.0, seed=rows, name="gate_pre")
    b = workloads.make_dense((rows, inter), act, seed=rows, name="up_pre")
    dh = workloads.make_dense((rows, inter), act, seed=rows, name="dh")
    c = moe.make_config(rows, 256, inter, 16, 4, 4, 2, 2, 1, act, act)
    da = torch.empty((rows, inter), dtype=a.dtype, device="cuda")
    db = torch.empty_like(da)
    moe.moe_swiglu_backward(c, a.cuda(), b.cuda(), dh.cuda(), rows, da, db)
    torch.cuda.synchronize()
    sel = workloads.sample_rows(rows, 256, seed=2).numpy()
    want_a, want_b = oracle.swiglu_backward(a[sel], b[sel], dh[sel])
    rel = 2.0 ** -8 if act == "bf16" else 2.0 ** -22
    for got, want in ((da.cpu()[sel].double().numpy(), want_a), (db.cpu()[sel].double().numpy(), want_b)):
        excess = np.abs(got - want) - rel * np.abs(want) - 1e-5 * np.abs(want).max()
        log(f"  max rel err {np.abs(got - want).max() / np.abs(want).max():.2e}")
        assert np.all(excess <= 0)


SMALL = dict(hidden=256, inter=256, E=16, K=4, G=4, M=2, topn=2)


@pytest.mark.parametrize("name,over", [("decode_bf16", dict(T=37, **SMALL)),
                                       ("decode_bf16", dict(T=64, Ns=0, **SMALL)),
                                       ("decode_bf16", dict(T=29, Ns=2, **SMALL)),
                                       ("decode_bf16", dict(T=1, **SMALL)),
                                       ("decode_bf16", dict(T=5, **{**SMALL, "K": 1, "M": 1})),
                                       ("decode_bf16", dict(T=400, **{**SMALL, "inter": 128})),
                                       ("decode_bf16", dict(T=50, **{**SMALL, "hidden": 128,
                                                                     "inter": 128})),
                                       # hidden 384, inter 640: partial last column tiles
                                       # of the [K][N]-weight GEMMs (dh: N = 640; dX:
                                       # N = 384, K = 1280 stacked at k_split = 640)
                                       ("decode_bf16", dict(T=90, **{**SMALL, "hidden": 384,
                                                                     "inter": 640})),
                                       ("decode_bf16", {})])
def test_expert_backward_input(name, over):
    """dx of the grouped SwiGLU experts against the oracle on up to 48 sampled tokens (the
    oracle run on those tokens' own rows); the oracle's routing and permutation are
    handed to the GPU.  Bound 2e-2 of the largest magnitude: the recomputed
    pre-activations, dh, da | db and the row gradients are each held in bf16."""
    from gpu_harness import config_of, expert_getter, inputs_on_gpu, oracle_route
    cfg = workloads.get(name).replace(**over)
    log(f"expert backward input {name} {over}")
    d = inputs_on_gpu(cfg)
    r = oracle_route(cfg, d)
    T, K, Ns, E, H = cfg.T, cfg.K, cfg.Ns, cfg.E, cfg.hidden
    load, off, row_token, pair_row = oracle.permute(r.idx, E)
    dy_rows = workloads.make_dense((cfg.rows, H), "bf16", seed=T, name="dy_rows")
    c = config_of(cfg)
    ws = torch.empty(moe.moe_backward_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()
    weights = {k: d[k] for k in ("w_gate", "w_up", "w_down")}
    moe.moe_expert_backward_input(c, d["x"], i32(off), i32(row_token), i32(pair_row), weights,
                                  dy_rows.cuda(), dx, ws)
    # a second micro-batch through the same workspace equals one through a fresh workspace
    # full of other bytes: nothing of an earlier call leaks into the next
    dy2 = workloads.make_dense((cfg.rows, H), "bf16", seed=T + 1, name="dy_rows")
    dx2 = torch.empty_like(dx)
    moe.moe_expert_backward_input(c, d["x"], i32(off), i32(row_token), i32(pair_row), weights,
                                  dy2.cuda(), dx2, ws)
    dx3 = torch.empty_like(dx)
    moe.moe_expert_backward_input(c, d["x"], i32(off), i32(row_token), i32(pair_row), weights,
                                  dy2.cuda(), dx3, torch.full_like(ws, 0x7f))
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx3), "the workspace's earlier contents changed the result"
    toks = workloads.sample_rows(T, 48, seed=4).numpy()
    n = len(toks)
    # the chosen tokens' rows, re-indexed as a problem of n tokens (routed, then shared)
    routed = pair_row.reshape(T, K)[toks].ravel()
    shared = np.concatenate([T * K + s * T + toks for s in range(Ns)]) if Ns else np.zeros(0, int)
    sub = np.concatenate([routed, shared]).astype(np.int64)
    expert_of_row = np.concatenate([np.searchsorted(off, routed, side="right") - 1,
                                    np.repeat(np.arange(E, E + Ns), n)])
    _, want = oracle.expert_input_backward(d["x"][toks], np.repeat(np.arange(n), K), n, K, Ns,
                                           dy_rows[sub], expert_getter(cfg, d), expert_of_row)
    got = dx.cpu()[toks].double().numpy()
    err = np.abs(got - want).max() / np.abs(want).max()
    log(f"  dx rel err {err:.2e} on {n} tokens")
    assert err <= 2e-2


@pytest.mark.parametrize("name,over,n_check", [("decode_bf16", dict(T=37, **SMALL), None),
                                               ("decode_bf16", dict(T=29, Ns=2, **SMALL), None),
                                               ("decode_bf16", dict(T=3, **SMALL), None),
                                               ("decode_bf16", dict(T=90, **{**SMALL, "hidden": 384,
                                                                             "inter": 640}), None),
                                               ("decode_bf16", {}, 4)])
def test_expert_backward_weights(name, over, n_check):
    """Weight gradients of every expert (small shapes) or of the shared expert and a few
    routed ones (full decode shape, among them one with no rows when there is one), and
    dx from the same call equal to moe_expert_backward_input's.  Bound 2e-2 of each
    matrix's largest magnitude (bf16 pre-activations and gradients, fp32 sums)."""
    from gpu_harness import config_of, expert_getter, inputs_on_gpu, oracle_route
    cfg = workloads.get(name).replace(**over)
    log(f"expert backward weights {name} {over}")
    d = inputs_on_gpu(cfg)
    r = oracle_route(cfg, d)
    T, K, Ns, E, H, I = cfg.T, cfg.K, cfg.Ns, cfg.E, cfg.hidden, cfg.inter
    load, off, row_token, pair_row = oracle.permute(r.idx, E)
    dy_rows = workloads.make_dense((cfg.rows, H), "bf16", seed=T + 7, name="dy_rows")
    c = config_of(cfg)
    ws = torch.empty(moe.moe_backward_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()
    weights = {k: d[k] for k in ("w_gate", "w_up", "w_down")}
    G = E + Ns
    dwg = torch.full((G, I, H), 7.0, device="cuda")
    dwu = torch.full((G, I, H), 7.0, device="cuda")
    dwd = torch.full((G, H, I), 7.0, device="cuda")
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dx_only = torch.empty_like(dx)
    args = (c, d["x"], i32(off), i32(row_token), i32(pair_row), weights, dy_rows.cuda())
    moe.moe_expert_backward(*args, dx, dwg, dwu, dwd, ws)
    moe.moe_expert_backward_input(*args, dx_only, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_only)
    expert_of_row = np.concatenate([np.repeat(np.arange(E), np.diff(off)),
                                    np.repeat(np.arange(E, G), T)])
    if n_check is None:
        check = list(range(G))
    else:
        empty = [e for e in range(E) if load[e] == 0][:1]
        busy = list(np.argsort(-load)[:n_check - len(empty)])
        check = sorted(set(empty + busy + list(range(E, G))))
    want = oracle.expert_weight_backward(d["x"], row_token, T, K, dy_rows, expert_getter(cfg, d),
                                         expert_of_row, check)
    worst = 0.0
    for e in check:
        for got, ref in zip((dwg[e], dwu[e], dwd[e]), want[e]):
            got = got.cpu().double().numpy()
            scale = np.abs(ref).max()
            if scale == 0.0:
                assert np.all(got == 0.0)
                continue
            worst = max(worst, np.abs(got - ref).max() / scale)
    log(f"  {len(check)} experts checked, worst rel err {worst:.2e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("name,over", [("decode_bf16", dict(T=37, **SMALL)),
                                       ("decode_bf16", dict(T=3, **SMALL)),
                                       ("decode_bf16", dict(T=700, **{**SMALL, "E": 72, "G": 8})),
                                       ("decode_bf16", dict(T=1000, E=250, G=10, M=4)),
                                       ("decode_bf16", {}),
                                       ("prefill_bf16", {})])
def test_router_backward(name, over):
    """dx = dz W_r (sampled tokens) and dW_r = dz^T x (all experts) against the oracle on
    a seeded logit gradient; bound 5e-5 of the largest magnitude: dz enters as two bf16
    parts (hi + lo within 2^-17 |dz|), products exact, fp32 sums over up to T = 8192
    terms (about eps * sqrt(T) relative to the result), with headroom.  Also the odd
    expert counts (padded to 64 inside) and token counts that leave ragged split-K
    ranges."""
    cfg = workloads.get(name).replace(**over)
    log(f"router backward {name} {over}")
    T, E, H = cfg.T, cfg.E, cfg.hidden
    x = workloads.make_tokens(cfg)
    w_r = workloads.make_router(cfg)
    dz = workloads.make_dense((T, E), "f32", std=1e-3, seed=T, name="grad_logits")
    from gpu_harness import config_of
    c = config_of(cfg)
    dx = torch.full((T, H), 7.0, device="cuda")
    dw = torch.full((E, H), 7.0, device="cuda")
    ws = torch.full((moe.moe_router_backward_workspace_bytes(c),), 0x7f, dtype=torch.uint8,
                    device="cuda")
    moe.moe_router_backward(c, x.cuda(), w_r.cuda(), dz.cuda(), dx, dw, ws)
    dx_only = torch.empty_like(dx)
    dw_only = torch.empty_like(dw)
    moe.moe_router_backward(c, x.cuda(), w_r.cuda(), dz.cuda(), dx_only, None, ws)
    moe.moe_router_backward(c, x.cuda(), w_r.cuda(), dz.cuda(), None, dw_only, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_only) and torch.equal(dw, dw_only)
    toks = workloads.sample_rows(T, 256, seed=6).numpy()
    want_dx, _ = oracle.router_backward(x[toks], w_r, dz[toks])
    _, want_dw = oracle.router_backward(x, w_r, dz)
    e_dx = np.abs(dx.cpu().double().numpy()[toks] - want_dx).max() / np.abs(want_dx).max()
    e_dw = np.abs(dw.cpu().double().numpy() - want_dw).max() / np.abs(want_dw).max()
    log(f"  dx rel err {e_dx:.2e}, dW_r rel err {e_dw:.2e}")
    assert e_dx <= 5e-5 and e_dw <= 5e-5


@pytest.mark.slow
def test_expert_backward_weights_prefill_rows():
    """Weight gradients at the prefill shape (T = 8192: the shared expert over 8192 rows,
    routed experts over about 256), in the launch the bench times, on 64 sampled
    intermediate channels i of the shared expert, the three busiest routed experts and
    the least busy one: rows i of dW_gate and dW_up, column i of dW_down.  The oracle
    runs each expert restricted to those channels (the SwiGLU is elementwise in i and
    dh_i needs only column i of W_down, so the restriction is the same computation)."""
    from gpu_harness import config_of, expert_getter, inputs_on_gpu, oracle_route
    cfg = workloads.get("prefill_bf16")
    log("expert backward weights at prefill rows (T=8192)")
    d = inputs_on_gpu(cfg)
    r = oracle_route(cfg, d)
    T, K, Ns, E, H, I = cfg.T, cfg.K, cfg.Ns, cfg.E, cfg.hidden, cfg.inter
    load, off, row_token, pair_row = oracle.permute(r.idx, E)
    dy_rows = workloads.make_dense((cfg.rows, H), "bf16", seed=11, name="dy_rows")
    c = config_of(cfg)
    ws = torch.empty(moe.moe_backward_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()
    weights = {k: d[k] for k in ("w_gate", "w_up", "w_down")}
    G = E + Ns
    dwg = torch.empty((G, I, H), device="cuda")
    dwu = torch.empty((G, I, H), device="cuda")
    dwd = torch.empty((G, H, I), device="cuda")
    moe.moe_expert_backward(c, d["x"], i32(off), i32(row_token), i32(pair_row), weights,
                            dy_rows.cuda(), None, dwg, dwu, dwd, ws)
    torch.cuda.synchronize()
    chan = np.sort(workloads.sample_rows(I, 64, seed=12).numpy())
    order = np.argsort(-load, kind="stable")
    check = [E] + [int(e) for e in order[:3]] + [int(order[-1])]
    log(f"  experts {check} with rows {[T] + [int(load[e]) for e in check[1:]]}")
    expert_of_row = np.concatenate([np.repeat(np.arange(E), np.diff(off)),
                                    np.repeat(np.arange(E, G), T)])
    full = expert_getter(cfg, d)
    get = lambda e: (lambda g, u, w: (g[chan], u[chan], w[:, chan]))(*full(e))
    worst = 0.0
    for e in check:
        want = oracle.expert_weight_backward(d["x"], row_token, T, K, dy_rows, get,
                                             expert_of_row, [e])[e]
        got = (dwg[e][chan], dwu[e][chan], dwd[e][:, chan])
        for gm, ref in zip(got, want):
            gm = gm.cpu().double().numpy()
            if np.abs(ref).max() == 0.0:               # an expert without rows
                assert np.all(gm == 0.0)
                continue
            worst = max(worst, np.abs(gm - ref).max() / np.abs(ref).max())
    log(f"  worst rel err {worst:.2e}")
    assert worst <= 2e-2
