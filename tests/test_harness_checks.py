"""The GPU tests' routing validity check (gpu_harness.check_routing) run on the host
with hand-made "GPU" outputs: valid alternatives pass, planted mistakes fail."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import check_routing


def _near_tie_case():
    cfg = workloads.get("tiny_fp32").replace(T=4, E=16, K=4, G=1, M=1, topn=1)
    s = np.tile(np.linspace(0.9, 0.15, 16), (4, 1))
    s[0, 4] = s[0, 3] - 5e-7                             # token 0: 3 and 4 tie at the K-th place
    r = oracle.select(s, np.zeros(16, np.float32), cfg.G, cfg.M, cfg.topn, cfg.K)
    return cfg, s, r


def _gates(s, idx):
    ss = np.take_along_axis(s, idx, 1)
    return ss / ss.sum(1, keepdims=True)


def test_canonical_and_valid_flip_pass():
    cfg, s, r = _near_tie_case()
    assert r.near_tie[0] and not r.near_tie[1:].any()
    idx = r.idx.copy()
    ref_idx, ref_gate, flipped = check_routing(cfg, r, torch.from_numpy(idx),
                                               torch.from_numpy(_gates(s, idx).astype(np.float32)))
    assert flipped == [] and np.array_equal(ref_idx, r.idx)
    idx[0, 3] = 4                                        # the other valid selection
    ref_idx, ref_gate, flipped = check_routing(cfg, r, torch.from_numpy(idx),
                                               torch.from_numpy(_gates(s, idx).astype(np.float32)))
    assert flipped == [0] and ref_idx[0].tolist() == [0, 1, 2, 4]
    np.testing.assert_allclose(ref_gate, _gates(s, idx), rtol=1e-15)


@pytest.mark.parametrize("mistake", ["far_expert", "order", "gate", "repeat", "other_token"])
def test_planted_mistakes_fail(mistake):
    cfg, s, r = _near_tie_case()
    idx = r.idx.copy()
    gate = _gates(s, idx).astype(np.float32)
    if mistake == "far_expert":
        idx[0, 3] = 9                                    # far below the K-th place
        gate = _gates(s, idx).astype(np.float32)
    elif mistake == "order":
        idx[1, [0, 1]] = idx[1, [1, 0]]
        gate = _gates(s, idx).astype(np.float32)
    elif mistake == "gate":
        gate[2, 0] *= 1.0001
    elif mistake == "repeat":
        idx[2, 1] = idx[2, 0]
    elif mistake == "other_token":
        idx[1, 3] = 4                                    # a flip where there is no near-tie
        gate = _gates(s, idx).astype(np.float32)
    with pytest.raises(AssertionError):
        check_routing(cfg, r, torch.from_numpy(idx), torch.from_numpy(gate))


def test_group_limit_is_enforced():
    cfg = workloads.get("tiny_fp32").replace(T=1, E=16, K=4, G=4, M=2, topn=2)
    s = np.full((1, 16), 0.2)
    s[0, [0, 1, 4, 5]] = [0.9, 0.8, 0.7, 0.6]           # groups 0 and 1
    r = oracle.select(s, np.zeros(16, np.float32), cfg.G, cfg.M, cfg.topn, cfg.K)
    idx = r.idx.copy()
    check_routing(cfg, r, torch.from_numpy(idx), torch.from_numpy(_gates(s, idx).astype(np.float32)))
    idx[0, 3] = 8                                        # a third group
    with pytest.raises(AssertionError):
        check_routing(cfg, r, torch.from_numpy(idx), torch.from_numpy(_gates(s, idx).astype(np.float32)))
