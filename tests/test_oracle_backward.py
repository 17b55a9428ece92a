"""Pins for the combine, gate and SwiGLU backward oracle (mathematics: the pages state the
forward formulas only)."""
import numpy as np
import pytest

import oracle


def _combine(Y, g, pair_row, T, K, Ns):
    """The forward combine written as plain loops (the map whose adjoint is pinned)."""
    out = np.zeros((T, Y.shape[1]))
    for t in range(T):
        for s in range(Ns):
            out[t] += Y[T * K + s * T + t]
        for k in range(K):
            out[t] += g[t, k] * Y[pair_row[t * K + k]]
    return out


def _case(seed, T=7, K=3, Ns=2, E=8, h=5):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, _, pair_row = oracle.permute(idx, E)
    rows = T * K + T * Ns
    return (rng.normal(size=(T, h)), rng.normal(size=(rows, h)), pair_row,
            rng.uniform(0.05, 1, size=(T, K)))


@pytest.mark.parametrize("seed,Ns", [(0, 2), (1, 0), (2, 1)])
def test_combine_adjoint_identity(seed, Ns):
    T, K = 7, 3
    dy, Y, pair_row, g = _case(seed, T=T, K=K, Ns=Ns)
    dgate, dY = oracle.combine_backward(dy, Y, pair_row, g, T, K, Ns)
    # C is linear in Y for fixed g: <dy, C(Y', g)> = <dY, Y'> for any Y'
    Y2 = np.random.default_rng(seed + 50).normal(size=Y.shape)
    np.testing.assert_allclose(np.sum(dy * _combine(Y2, g, pair_row, T, K, Ns)), np.sum(dY * Y2),
                               rtol=1e-12)
    # and its routed part is linear in g for fixed Y: <dy, C(Y, g') - C(Y, 0)> = <dg, g'>
    g2 = np.random.default_rng(seed + 60).normal(size=g.shape)
    lhs = np.sum(dy * (_combine(Y, g2, pair_row, T, K, Ns) - _combine(Y, 0 * g2, pair_row, T, K, Ns)))
    np.testing.assert_allclose(lhs, np.sum(dgate * g2), rtol=1e-12)


def test_combine_backward_hand_computed():
    # T = 1, K = 2, Ns = 1, h = 2: rows 0, 1 routed (pair (0,0) -> row 1, (0,1) -> row 0),
    # row 2 shared.  dy = [1, 2]; Y[0] = [3, -1], Y[1] = [0.5, 4]; g = [0.25, 0.75]
    # dg = [<dy, Y[1]>, <dy, Y[0]>] = [8.5, 1]; dY[1] = 0.25 dy, dY[0] = 0.75 dy, dY[2] = dy
    dy = np.array([[1.0, 2.0]])
    Y = np.array([[3.0, -1.0], [0.5, 4.0], [9.0, 9.0]])
    dgate, dY = oracle.combine_backward(dy, Y, np.array([1, 0]), np.array([[0.25, 0.75]]), 1, 2, 1)
    np.testing.assert_array_equal(dgate, [[8.5, 1.0]])
    np.testing.assert_array_equal(dY, [[0.75, 1.5], [0.25, 0.5], [1.0, 2.0]])


@pytest.mark.parametrize("seed,T,E,K", [(3, 5, 8, 3), (4, 4, 16, 4), (5, 3, 4, 1)])
def test_gate_backward_matches_central_differences(seed, T, E, K):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1.5, size=(T, E))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    dg = rng.normal(size=(T, K))

    def loss(zz):
        s = 1.0 / (1.0 + np.exp(-zz))
        sel = np.take_along_axis(s, idx, 1)
        return np.sum(dg * sel / sel.sum(1, keepdims=True))

    grad = oracle.gate_backward(z, idx, dg)
    h = 1e-6
    fd = np.zeros_like(z)
    for t in range(T):
        for e in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, e] += h
            zm[t, e] -= h
            fd[t, e] = (loss(zp) - loss(zm)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-10)
    # unselected experts get exactly zero (no path from their logits to the gates)
    mask = np.ones_like(z, bool)
    np.put_along_axis(mask, idx, False, axis=1)
    assert np.all(grad[mask] == 0.0)


def test_gate_backward_hand_computed_and_closed_form():
    # K = 2, z = 0 on both selected experts: s = 1/2, S = 1, g = [1/2, 1/2];
    # dg = [1, 0]: ds = (dg - <dg, g>) / S = [1/2, -1/2]; dz = ds * s (1 - s) = [1/8, -1/8]
    z = np.zeros((1, 4))
    grad = oracle.gate_backward(z, np.array([[2, 0]]), np.array([[1.0, 0.0]]))
    np.testing.assert_allclose(grad, [[-0.125, 0.0, 0.125, 0.0]], rtol=0, atol=1e-15)
    # a gradient equal over the selection moves nothing: the gates always sum to one
    rng = np.random.default_rng(9)
    z = rng.normal(size=(6, 16))
    idx = np.stack([rng.choice(16, 4, replace=False) for _ in range(6)])
    g = oracle.gate_backward(z, idx, np.full((6, 4), 3.7))
    np.testing.assert_allclose(g, 0.0, atol=1e-15)


def test_swiglu_backward_matches_central_differences():
    rng = np.random.default_rng(11)
    a = rng.normal(0, 2, size=(4, 6))
    b = rng.normal(size=(4, 6))
    dh = rng.normal(size=(4, 6))

    def loss(aa, bb):
        return np.sum(dh * aa / (1.0 + np.exp(-aa)) * bb)

    da, db = oracle.swiglu_backward(a, b, dh)
    h = 1e-6
    for i in range(4):
        for j in range(6):
            e = np.zeros_like(a)
            e[i, j] = h
            np.testing.assert_allclose(da[i, j], (loss(a + e, b) - loss(a - e, b)) / (2 * h),
                                       rtol=1e-6, atol=1e-9)
            np.testing.assert_allclose(db[i, j], (loss(a, b + e) - loss(a, b - e)) / (2 * h),
                                       rtol=1e-6, atol=1e-9)


def test_swiglu_backward_closed_forms():
    # at a = 0: sigmoid = 1/2, silu = 0, silu' = 1/2 -> da = dh b / 2, db = 0
    b = np.array([[2.0, -3.0]])
    dh = np.array([[0.5, 4.0]])
    da, db = oracle.swiglu_backward(np.zeros((1, 2)), b, dh)
    np.testing.assert_array_equal(da, [[0.5, -6.0]])
    np.testing.assert_array_equal(db, [[0.0, 0.0]])
    # far positive a: silu(a) -> a and silu'(a) -> 1
    da, db = oracle.swiglu_backward(np.array([[40.0]]), np.array([[3.0]]), np.array([[2.0]]))
    np.testing.assert_allclose(da, [[6.0]], rtol=1e-12)
    np.testing.assert_allclose(db, [[80.0]], rtol=1e-12)


def _ffn_case(seed, T=4, K=2, Ns=1, E=3, H=5, I=4):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    _, off, row_token, _ = oracle.permute(idx, E)
    experts = [(rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I)))
               for _ in range(E + Ns)]
    rows = T * K + T * Ns
    expert_of_row = np.concatenate([np.repeat(np.arange(E), np.diff(off)),
                                    np.repeat(np.arange(E, E + Ns), T)])
    return rng.normal(size=(T, H)), row_token, experts, expert_of_row, rng.normal(size=(rows, H))


def test_expert_input_backward_matches_central_differences():
    T, K, Ns = 4, 2, 1
    x, row_token, experts, eor, dY = _ffn_case(12, T=T, K=K, Ns=Ns)
    tok = [row_token[r] if r < T * K else (r - T * K) % T for r in range(len(eor))]

    def loss(xx):
        total = 0.0
        for r, e in enumerate(eor):
            total += np.dot(dY[r], oracle.expert_ffn(xx[tok[r]][None, :], *experts[e])[0])
        return total

    dX, dx = oracle.expert_input_backward(x, row_token, T, K, Ns, dY, lambda e: experts[e], eor)
    h = 1e-6
    for t in range(T):
        for c in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[t, c] += h
            xm[t, c] -= h
            np.testing.assert_allclose(dx[t, c], (loss(xp) - loss(xm)) / (2 * h), rtol=1e-6,
                                       atol=1e-8)
    # linear in dy: doubling one row's gradient doubles that row's dX only
    dY2 = dY.copy()
    dY2[3] *= 2
    dX2, _ = oracle.expert_input_backward(x, row_token, T, K, Ns, dY2, lambda e: experts[e], eor)
    np.testing.assert_allclose(dX2[3], 2 * dX[3], rtol=1e-12)
    np.testing.assert_allclose(np.delete(dX2, 3, 0), np.delete(dX, 3, 0), rtol=0, atol=0)


def test_expert_weight_backward_matches_central_differences():
    T, K, Ns = 4, 2, 1
    x, row_token, experts, eor, dY = _ffn_case(13, T=T, K=K, Ns=Ns)
    tok = [row_token[r] if r < T * K else (r - T * K) % T for r in range(len(eor))]

    def loss(ex):
        return sum(np.dot(dY[r], oracle.expert_ffn(x[tok[r]][None, :], *ex[e])[0])
                   for r, e in enumerate(eor))

    grads = oracle.expert_weight_backward(x, row_token, T, K, dY, lambda e: experts[e], eor,
                                          range(len(experts)))
    h = 1e-6
    for e in range(len(experts)):
        for m in range(3):                   # gate, up, down
            W = experts[e][m]
            for idx in [(0, 0), (1, 2), (W.shape[0] - 1, W.shape[1] - 1)]:
                plus = [list(t) for t in experts]
                minus = [list(t) for t in experts]
                Wp, Wm = W.copy(), W.copy()
                Wp[idx] += h
                Wm[idx] -= h
                plus[e][m], minus[e][m] = Wp, Wm
                fd = (loss(plus) - loss(minus)) / (2 * h)
                np.testing.assert_allclose(grads[e][m][idx], fd, rtol=1e-6, atol=1e-8)


def test_router_backward_adjoint_identities():
    rng = np.random.default_rng(14)
    x, w, dz = rng.normal(size=(6, 5)), rng.normal(size=(4, 5)), rng.normal(size=(6, 4))
    dx, dw = oracle.router_backward(x, w, dz)
    x2, w2 = rng.normal(size=x.shape), rng.normal(size=w.shape)
    np.testing.assert_allclose(np.sum(dz * (x2 @ w.T)), np.sum(dx * x2), rtol=1e-12)
    np.testing.assert_allclose(np.sum(dz * (x @ w2.T)), np.sum(dw * w2), rtol=1e-12)
    # hand case: one token, one expert: z = <x, w>, dz = 2 -> dx = 2 w, dW = 2 x
    dx1, dw1 = oracle.router_backward(np.array([[1.0, -2.0]]), np.array([[3.0, 0.5]]),
                                      np.array([[2.0]]))
    np.testing.assert_array_equal(dx1, [[6.0, 1.0]])
    np.testing.assert_array_equal(dw1, [[2.0, -4.0]])

