"""Pins for the routing oracle (affinity, bias, group limit, top-K, gates).

The oracle is checked against things other than itself:
  * brute-force enumeration of every group subset and every expert subset,
  * torch.topk when the group limit is inactive (M = G),
  * invariants the pages fix: K distinct experts, at most M groups touched,
    gates positive and summing to 1, the bias changes selection but not gate
    values, a constant bias shift changes nothing, b = 0 and M = G is top-K of z,
  * planted exact ties (lower index wins).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def _rand_case(rng, T, E, h, bias_scale):
    x = rng.standard_normal((T, h)).astype(np.float32)
    w = (0.3 * rng.standard_normal((E, h))).astype(np.float32)
    b = (bias_scale * rng.standard_normal(E)).astype(np.float32)
    return x, w, b


def _brute_force(sb_row, G, M, topn, K):
    """Two-stage selection by exhaustive enumeration (float64 biased affinities)."""
    E = sb_row.shape[0]
    n = E // G
    # a group's score: the best sum over all topn-subsets of its experts
    gscore = [max(sum(c) for c in itertools.combinations(sb_row[j * n:(j + 1) * n], topn))
              for j in range(G)]
    # stage 1: the M-subset of groups with the largest total score
    best_groups = max(itertools.combinations(range(G), M), key=lambda c: sum(gscore[j] for j in c))
    cand = [e for j in best_groups for e in range(j * n, (j + 1) * n)]
    # stage 2: the K-subset of candidates with the largest total biased affinity
    best = max(itertools.combinations(cand, K), key=lambda c: sum(sb_row[e] for e in c))
    return set(best_groups), set(best)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("E,G,M,topn,K", [(16, 4, 2, 2, 4), (12, 3, 2, 2, 3), (16, 8, 3, 2, 5),
                                          (16, 2, 1, 3, 4)])
def test_route_matches_brute_force(seed, E, G, M, topn, K):
    rng = np.random.default_rng(seed)
    x, w, b = _rand_case(rng, 24, E, 32, 0.05)
    r = oracle.route(x, w, b, G, M, topn, K)
    checked = 0
    for t in range(x.shape[0]):
        if r.near_tie[t]:
            continue
        groups, sel = _brute_force(r.sb[t], G, M, topn, K)
        assert set(r.groups[t].tolist()) == groups
        assert set(r.idx[t].tolist()) == sel
        checked += 1
    assert checked >= 20


def test_bias_changes_group_choice_like_brute_force():
    """A bias that flips which groups win: the group score must use biased affinities."""
    rng = np.random.default_rng(7)
    x, w, _ = _rand_case(rng, 16, 16, 32, 0.0)
    b = np.zeros(16, np.float32)
    b[12:16] = 0.6          # lift group 3 in selection only
    r = oracle.route(x, w, b, 4, 2, 2, 4)
    for t in range(16):
        assert 3 in r.groups[t].tolist()
        groups, sel = _brute_force(r.sb[t], 4, 2, 2, 4)
        assert set(r.groups[t].tolist()) == groups and set(r.idx[t].tolist()) == sel


@pytest.mark.parametrize("seed", [0, 3])
def test_no_group_limit_is_torch_topk(seed):
    rng = np.random.default_rng(seed)
    x, w, b = _rand_case(rng, 64, 32, 48, 0.02)
    r = oracle.route(x, w, b, 4, 4, 2, 6)          # M = G: every group kept
    ref = torch.topk(torch.from_numpy(r.sb), 6, dim=1, sorted=True).indices.numpy()
    ok = ~r.near_tie & ~r.near_tie_order
    assert ok.sum() > 50
    np.testing.assert_array_equal(r.idx[ok], ref[ok])


def test_zero_bias_no_limit_is_topk_of_logits():
    rng = np.random.default_rng(11)
    x, w, _ = _rand_case(rng, 64, 16, 40, 0.0)
    r = oracle.route(x, w, np.zeros(16, np.float32), 1, 1, 2, 4)   # G = 1
    z = x.astype(np.float64) @ w.astype(np.float64).T
    ref = np.argsort(-z, axis=1, kind="stable")[:, :4]
    ok = ~r.near_tie & ~r.near_tie_order
    np.testing.assert_array_equal(r.idx[ok], ref[ok])


def test_invariants_full_shape():
    """256 experts, 8 groups, M = 4, top-8, biased; a few tokens at full width."""
    rng = np.random.default_rng(5)
    T, E, h, G, M, K = 48, 256, 256, 8, 4, 8
    x = rng.standard_normal((T, h)).astype(np.float32)
    w = (0.02 * 8 * rng.standard_normal((E, h))).astype(np.float32)
    b = rng.uniform(-0.01, 0.01, E).astype(np.float32)
    r = oracle.route(x, w, b, G, M, 2, K)
    for t in range(T):
        sel = r.idx[t].tolist()
        assert len(set(sel)) == K
        assert len({e // (E // G) for e in sel}) <= M
        assert set(e // (E // G) for e in sel) <= set(r.groups[t].tolist())
        # ordered by (biased affinity desc, index asc)
        keys = [(-r.sb[t, e], e) for e in sel]
        if not r.near_tie_order[t]:
            assert keys == sorted(keys)
    assert np.all(r.gate > 0)
    np.testing.assert_allclose(r.gate.sum(1), 1.0, rtol=0, atol=1e-12)
    # gates are s / sum(s) over the chosen set, independent of the bias
    s_sel = np.take_along_axis(r.s, r.idx.astype(np.int64), 1)
    np.testing.assert_allclose(r.gate, s_sel / s_sel.sum(1, keepdims=True), rtol=1e-15)


def test_bias_selects_but_does_not_gate():
    rng = np.random.default_rng(9)
    x, w, _ = _rand_case(rng, 32, 16, 32, 0.0)
    r0 = oracle.route(x, w, np.zeros(16, np.float32), 4, 2, 2, 4)
    b = np.zeros(16, np.float32)
    b[r0.idx[0, 0]] = -1.0           # forbid token 0's best expert in selection
    r1 = oracle.route(x, w, b, 4, 2, 2, 4)
    assert r0.idx[0, 0] not in r1.idx[0].tolist()
    # for every token whose chosen set did not change, gates are identical
    same = [t for t in range(32) if set(r0.idx[t]) == set(r1.idx[t])]
    assert len(same) > 10
    for t in same:
        g0 = dict(zip(r0.idx[t].tolist(), r0.gate[t].tolist()))
        g1 = dict(zip(r1.idx[t].tolist(), r1.gate[t].tolist()))
        assert g0 == g1


def test_constant_bias_shift_is_noop():
    rng = np.random.default_rng(13)
    x, w, b = _rand_case(rng, 64, 16, 32, 0.05)
    r0 = oracle.route(x, w, b, 4, 2, 2, 4)
    r1 = oracle.route(x, w, (b + np.float32(0.125)).astype(np.float32), 4, 2, 2, 4)
    ok = ~(r0.near_tie | r1.near_tie)
    assert ok.sum() > 50
    for t in np.nonzero(ok)[0]:
        assert set(r0.idx[t]) == set(r1.idx[t])
    np.testing.assert_allclose(np.sort(r0.gate[ok], 1), np.sort(r1.gate[ok], 1), rtol=1e-15)


def test_exact_ties_go_to_lower_index():
    # identical router rows give identical affinities: experts 1 and 2 tie exactly
    h = 8
    x = np.ones((1, h), np.float32)
    w = np.zeros((4, h), np.float32)
    w[0] = 0.5
    w[1] = 0.25
    w[2] = 0.25
    w[3] = -0.5
    r = oracle.route(x, w, np.zeros(4, np.float32), 1, 1, 2, 2)
    assert r.idx[0].tolist() == [0, 1]
    # tied groups: groups {0,1} and {2,3} with equal scores -> group 0 kept
    w2 = np.zeros((4, h), np.float32)
    w2[0] = w2[2] = 0.3
    w2[1] = w2[3] = 0.1
    r2 = oracle.route(x, w2, np.zeros(4, np.float32), 2, 1, 2, 2)
    assert r2.groups[0].tolist() == [0] and r2.idx[0].tolist() == [0, 1]
    assert r2.near_tie_group[0]


def test_near_tie_flag_on_planted_gap():
    h = 4
    x = np.ones((1, h), np.float32)
    w = np.zeros((3, h), np.float32)
    w[0] = 0.5
    w[1] = 0.2
    w[2] = 0.2
    b = np.array([0.0, 0.0, 5e-7], np.float32)      # expert 2 ahead of 1 by 5e-7
    r = oracle.route(x, w, b, 1, 1, 1, 2)
    assert r.idx[0].tolist() == [0, 2]
    assert r.near_tie_expert[0]


def _valid_brute(sb_row, G, M, topn, K, tol=1e-6):
    """Every K-set that is a top-K (within tol) of some top-M group set (within tol), by
    enumerating all group subsets and all expert subsets."""
    E = sb_row.shape[0]
    n = E // G
    gscore = [sum(sorted(sb_row[j * n:(j + 1) * n], reverse=True)[:topn]) for j in range(G)]
    out = set()
    for S in itertools.combinations(range(G), M):
        rest_g = [gscore[j] for j in range(G) if j not in S]
        if rest_g and min(gscore[j] for j in S) < max(rest_g) - tol:
            continue
        cand = [e for j in S for e in range(j * n, (j + 1) * n)]
        for X in itertools.combinations(cand, K):
            rest = [sb_row[e] for e in cand if e not in X]
            if not rest or min(sb_row[e] for e in X) >= max(rest) - tol:
                out.add(frozenset(X))
    return out


@pytest.mark.parametrize("E,G,M,topn,K", [(16, 4, 2, 2, 4), (12, 3, 2, 2, 3), (8, 4, 4, 1, 3),
                                          (8, 1, 1, 1, 2), (16, 8, 3, 2, 5)])
def test_valid_selections_brute_force(E, G, M, topn, K):
    """Affinities on a coarse grid (steps of 4e-7 around three levels) so that many
    tokens have several valid selections; the enumeration equals brute force, always
    holds the canonical selection, and is that selection alone without near-ties."""
    rng = np.random.default_rng(E * 100 + K)
    multi = 0
    for t in range(60):
        sb = 0.5 + 0.1 * rng.integers(0, 3, E) + 4e-7 * rng.integers(0, 4, E)
        want = _valid_brute(sb, G, M, topn, K)
        got = oracle.valid_selections(sb, G, M, topn, K)
        assert got == want, t
        r = oracle.select(sb[None, :] - 0.0, np.zeros(E, np.float32), G, M, topn, K)
        assert frozenset(r.idx[0].tolist()) in got
        if not r.near_tie[0]:
            assert got == {frozenset(r.idx[0].tolist())}
        multi += len(got) > 1
    assert multi >= 5
    # a planted flip: two experts 5e-7 apart straddle the K-th place
    sb = np.linspace(0.9, 0.1, E)
    sb[K] = sb[K - 1] - 5e-7
    got = oracle.valid_selections(sb, 1, 1, 1, K)
    top = list(range(K))
    assert got == {frozenset(top), frozenset(top[:-1] + [K])}
