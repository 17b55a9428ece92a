"""Pins for the sequence-wise balance loss oracle (mathematics; the pages print no
formula and no worked example of it)."""
import numpy as np
import pytest

import oracle

ALPHA = 1e-4


def test_hand_computed_normalised_rows():
    # E = 4, K = 1, one sequence of 2 tokens; rows already sum to 1 (s' = s).
    # counts [1, 1, 0, 0] -> f = 4 / (1 * 2) * counts = [2, 2, 0, 0]
    # P = column means = [0.65, 0.2, 0.075, 0.075]; L = alpha (2*0.65 + 2*0.2) = 1.7 alpha
    s = np.array([[0.8, 0.1, 0.05, 0.05], [0.5, 0.3, 0.1, 0.1]])
    idx = np.array([[0], [1]])
    loss, f, P = oracle.balance_loss(s, idx, 2, ALPHA, 1)
    np.testing.assert_allclose(f[0], [2, 2, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(P[0], [0.65, 0.2, 0.075, 0.075], rtol=0, atol=1e-15)
    np.testing.assert_allclose(loss, [1.7 * ALPHA], rtol=1e-14)


def test_hand_computed_unnormalised_rows():
    # row 0 sums to 2 -> s' = [0.4, 0.4, 0.1, 0.1]; row 1 sums to 1 -> s' = s.
    # K = 2: token 0 picks {0, 1}, token 1 picks {2, 0}: counts [2, 1, 1, 0],
    # f = 4 / (2 * 2) * counts = [2, 1, 1, 0]; P = [0.35, 0.25, 0.2, 0.2];
    # L = alpha (0.7 + 0.25 + 0.2) = 1.15 alpha
    s = np.array([[0.8, 0.8, 0.2, 0.2], [0.3, 0.1, 0.3, 0.3]])
    idx = np.array([[0, 1], [2, 0]])
    loss, f, P = oracle.balance_loss(s, idx, 2, ALPHA, 2)
    np.testing.assert_allclose(f[0], [2, 1, 1, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(P[0], [0.35, 0.25, 0.2, 0.2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(loss, [1.15 * ALPHA], rtol=1e-14)


def _random_case(seed, T, E, K):
    rng = np.random.default_rng(seed)
    s = 1.0 / (1.0 + np.exp(-rng.normal(0, 1.7, size=(T, E))))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    return s, idx


def test_perfect_balance_gives_alpha_for_any_affinities():
    # every expert chosen T_s K / E times in each sequence -> f = 1 -> L = alpha sum P = alpha
    T, E, K, L = 32, 16, 4, 8
    idx = np.array([[(K * t + k) % E for k in range(K)] for t in range(T)])
    s, _ = _random_case(0, T, E, K)
    loss, f, _ = oracle.balance_loss(s, idx, L, ALPHA, K)
    np.testing.assert_allclose(f, 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(loss, ALPHA, rtol=1e-13)


def test_uniform_affinities_give_alpha_for_any_selection():
    # s' = 1/E everywhere -> L = alpha / E * sum f = alpha (sum f = E)
    T, E, K = 24, 16, 4
    _, idx = _random_case(1, T, E, K)
    loss, _, P = oracle.balance_loss(np.full((T, E), 0.3), idx, 12, ALPHA, K)
    np.testing.assert_allclose(P, 1.0 / E, rtol=1e-14)
    np.testing.assert_allclose(loss, ALPHA, rtol=1e-13)


def test_full_concentration_reaches_the_bound():
    # all tokens pick experts 0..K-1 and put all their affinity there:
    # f_i = E/K on them, sum of their P = 1 -> L = alpha E / K (the maximum)
    T, E, K = 16, 16, 4
    s = np.zeros((T, E))
    s[:, :K] = 0.7
    idx = np.tile(np.arange(K), (T, 1))
    loss, _, _ = oracle.balance_loss(s, idx, 8, ALPHA, K)
    np.testing.assert_allclose(loss, ALPHA * E / K, rtol=1e-13)


@pytest.mark.parametrize("seed,T,E,K,L", [(2, 48, 16, 4, 12), (3, 64, 256, 8, 64), (4, 10, 8, 3, 5)])
def test_invariants(seed, T, E, K, L):
    s, idx = _random_case(seed, T, E, K)
    loss, f, P = oracle.balance_loss(s, idx, L, ALPHA, K)
    np.testing.assert_allclose(f.sum(axis=1), E, rtol=1e-13)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-13)
    assert np.all(loss > 0) and np.all(loss <= ALPHA * E / K * (1 + 1e-12))
    # relabelling the experts changes nothing
    perm = np.random.default_rng(seed + 100).permutation(E)
    inv = np.argsort(perm)                       # new label of old expert e is inv[e]
    s2 = s[:, perm]                              # column j of s2 is old expert perm[j]
    loss2, f2, P2 = oracle.balance_loss(s2, inv[idx], L, ALPHA, K)
    np.testing.assert_allclose(loss2, loss, rtol=1e-12)
    np.testing.assert_allclose(f2, f[:, perm], rtol=1e-13)
    # each sequence's loss depends only on its own tokens
    for q in range(T // L):
        rows = slice(q * L, (q + 1) * L)
        lq, _, _ = oracle.balance_loss(s[rows], idx[rows], L, ALPHA, K)
        np.testing.assert_allclose(lq, loss[q:q + 1], rtol=1e-13)


def test_batch_wise_is_one_sequence_and_scale_of_alpha():
    s, idx = _random_case(5, 40, 16, 4)
    batch, fb, Pb = oracle.balance_loss(s, idx, 40, 1.0, 4)
    seq, fs, Ps = oracle.balance_loss(s, idx, 10, 1.0, 4)
    # f and P are linear averages: the batch's are the means of the sequences'
    np.testing.assert_allclose(fb[0], fs.mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(Pb[0], Ps.mean(axis=0), rtol=1e-13)
    scaled, _, _ = oracle.balance_loss(s, idx, 40, 3.0, 4)
    np.testing.assert_allclose(scaled, 3.0 * batch, rtol=1e-14)


@pytest.mark.parametrize("seed,T,E,K,L", [(6, 6, 8, 2, 3), (7, 8, 16, 4, 8)])
def test_gradient_matches_central_differences(seed, T, E, K, L):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1.5, size=(T, E))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    alpha = 0.1

    def total(zz):
        return oracle.balance_loss(1.0 / (1.0 + np.exp(-zz)), idx, L, alpha, K)[0].sum()

    g = oracle.balance_loss_grad_logits(z, idx, L, alpha, K)
    h = 1e-6
    fd = np.zeros_like(z)
    for t in range(T):
        for e in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, e] += h
            zm[t, e] -= h
            fd[t, e] = (total(zp) - total(zm)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-10)
    # with perfect balance f = 1 for every expert, so f_j - sum_i f_i s'_i = 0: no gradient
    idx_bal = np.array([[(K * t + k) % E for k in range(K)] for t in range(E // K * 2)])
    zb = rng.normal(0, 1.5, size=idx_bal.shape[:1] + (E,))
    gb = oracle.balance_loss_grad_logits(zb, idx_bal, idx_bal.shape[0], alpha, K)
    np.testing.assert_allclose(gb, 0.0, atol=1e-15)
