"""moe_layer_forward_noalloc (the workspace held by the library, for callers that
cannot allocate) against moe_layer_forward with a caller workspace: two calls in a
row on one device, the second on a smaller batch, each bit-identical to the
workspace entry point (the same kernels in the same order), and a batch whose
workspace exceeds the library's array rejected before anything runs."""
import pytest
import torch

import sparse_moe_layer_affinity_amd as moe
import workloads
from gpu_harness import config_of, inputs_on_gpu, layer_forward, log, weights_of

pytestmark = pytest.mark.gpu


def _noalloc(cfg, d):
    c = config_of(cfg)
    out = {
        "y": torch.empty((cfg.T, cfg.hidden), dtype=torch.bfloat16, device="cuda"),
        "idx": torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda"),
        "gate": torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda"),
        "load": torch.empty(cfg.E, dtype=torch.int32, device="cuda"),
    }
    moe.moe_layer_forward_noalloc(c, d["x"], d["w_router"], d["bias"], weights_of(d), None,
                                  out["y"], out["idx"], out["gate"], out["load"])
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_workspace_entry():
    big = workloads.get("decode_bf16")                                    # T = 128, h = 7168
    small = workloads.get("prefill_fp8").replace(T=37, hidden=256, inter=256, E=16, K=4, G=4,
                                                 M=2, compare_rows=None)
    for cfg in (big, small):
        log(f"noalloc layer forward {cfg.name} T={cfg.T} ({cfg.w})")
        d = inputs_on_gpu(cfg)
        got = _noalloc(cfg, d)
        want = layer_forward(cfg, d)
        for k in ("y", "idx", "gate", "load"):
            assert torch.equal(got[k], want[k]), f"{cfg.name}: {k} differs"
    # the same small batch again right after: the array keeps the last call's contents
    again = _noalloc(small, d)
    for k in ("y", "idx", "gate", "load"):
        assert torch.equal(again[k], want[k]), f"repeat: {k} differs"


def test_noalloc_rejects_large_batches():
    cfg = workloads.get("prefill_bf16")                                   # T = 8192
    c = config_of(cfg)
    assert moe.moe_workspace_bytes(c) > 64 << 20
    dummy = torch.empty(16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(c, dummy, dummy, dummy, {"w_gate": dummy, "w_up": dummy,
                                                               "w_down": dummy},
                                      None, dummy, dummy, dummy, dummy)
    assert e.value.code == 2                                              # MOE_ERR_UNSUPPORTED
