"""Pins for the permutation (no token dropping) and the aux-loss-free bias update."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _loops_permute(idx, E):
    """Plain loops: walk experts in order, and tokens in order within an expert."""
    T, K = idx.shape
    load = [0] * E
    row_token, pair_row = [], [None] * (T * K)
    for e in range(E):
        for t in range(T):
            for k in range(K):
                if idx[t, k] == e:
                    pair_row[t * K + k] = len(row_token)
                    row_token.append(t)
                    load[e] += 1
    return np.array(load), np.array(row_token), np.array(pair_row)


@pytest.mark.parametrize("seed,T,E,K", [(0, 37, 16, 4), (1, 5, 8, 3), (2, 64, 256, 8), (3, 1, 4, 2)])
def test_permute_matches_loops(seed, T, E, K):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    load, off, row_token, pair_row = oracle.permute(idx, E)
    l2, rt2, pr2 = _loops_permute(idx, E)
    np.testing.assert_array_equal(load, l2)
    np.testing.assert_array_equal(row_token, rt2)
    np.testing.assert_array_equal(pair_row, pr2)
    assert off[0] == 0 and off[-1] == T * K and np.all(np.diff(off) == load)
    assert sorted(pair_row.tolist()) == list(range(T * K))          # a bijection
    np.testing.assert_array_equal(row_token[pair_row], np.repeat(np.arange(T), K))


def test_permute_skewed_and_empty_experts():
    idx = np.array([[0, 1], [0, 2], [0, 1], [3, 0]], np.int32)
    load, off, row_token, pair_row = oracle.permute(idx, 6)
    assert load.tolist() == [4, 2, 1, 1, 0, 0]
    assert off.tolist() == [0, 4, 6, 7, 8, 8, 8]
    assert row_token.tolist() == [0, 1, 2, 3, 0, 2, 1, 3]
    assert pair_row.tolist() == [0, 4, 1, 6, 2, 5, 7, 3]


def _read_golden_bias():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "bias_update.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, val = line.split("=", 1)
            key = key.strip()
            if key == "case":
                cur = {}
                cases.append(cur)
            else:
                cur[key] = [float(v) for v in val.split()]
    return cases


def test_bias_update_golden():
    for c in _read_golden_bias():
        T, K = int(c["T"][0]), int(c["K"][0])
        got = oracle.bias_update(np.array(c["load"], np.int64), np.array(c["bias"], np.float32),
                                 c["gamma"][0], T, K)
        np.testing.assert_array_equal(got, np.array(c["expected"], np.float32))


def test_bias_update_closed_form():
    rng = np.random.default_rng(0)
    E, T, K = 256, 8192, 8
    load = rng.multinomial(T * K, np.ones(E) / E)
    load[:4] = T * K // E                           # exactly at the mean: unchanged
    b = rng.uniform(-0.01, 0.01, E).astype(np.float32)
    nb = oracle.bias_update(load, b, 1e-3, T, K)
    assert nb.dtype == np.float32
    g = np.float32(1e-3)
    for e in range(E):
        if load[e] * E > T * K:
            assert nb[e] < b[e] and nb[e] == np.float32(b[e] - g)
        elif load[e] * E < T * K:
            assert nb[e] > b[e] and nb[e] == np.float32(b[e] + g)
        else:
            assert nb[e] == b[e]
    # |delta| is gamma up to one float32 rounding
    d = np.abs(nb.astype(np.float64) - b.astype(np.float64))
    assert np.all((d == 0) | (np.abs(d - 1e-3) < 1e-8))


def test_bias_update_drives_balance():
    """Repeated updates against fixed per-expert preferences shrink the max/mean load."""
    rng = np.random.default_rng(1)
    T, E, K, h = 512, 16, 2, 32
    x = rng.standard_normal((T, h)).astype(np.float32)
    w = (0.2 * rng.standard_normal((E, h))).astype(np.float32)
    w[:, 0] = 0.0
    w[0, 0] = 3.0
    x[:, 0] = 1.0
    b = np.zeros(E, np.float32)
    ratios = []
    for _ in range(60):
        r = oracle.route(x, w, b, 4, 2, 2, K)
        load, *_ = oracle.permute(r.idx, E)
        ratios.append(load.max() / (T * K / E))
        b = oracle.bias_update(load, b, 2e-2, T, K)
    assert ratios[0] > 4.0
    assert ratios[-1] < 0.5 * ratios[0]
