"""Host-only checks of the C ABI: the library loads, exports every declared entry
point, and rejects invalid arguments with the documented status before any launch.
No call here reaches a kernel launch, so no GPU is needed."""
import ctypes
import subprocess

import pytest

import sparse_moe_layer_affinity_amd as moe
from sparse_moe_layer_affinity_amd import binding as B

ALIGNED = 1 << 20          # a fake, 256-byte aligned address: never dereferenced here


def cfg(**kw):
    base = dict(T=8192, hidden=7168, inter=2048, E=256, K=8, G=8, M=4, topn=2, Ns=1,
                act="bf16", w="bf16")
    base.update(kw)
    return B.make_config(**base)


def code_of(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except B.MoeError as e:
        return e.code
    return B.MOE_OK


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = B.header_symbols()
    assert set(names) == {"moe_workspace_bytes", "moe_route", "moe_permute", "moe_act_quant_e4m3",
                          "moe_grouped_ffn", "moe_combine", "moe_bias_update", "moe_layer_forward",
                          "moe_router_scores", "moe_balance_loss", "moe_combine_backward",
                          "moe_gate_backward", "moe_swiglu_backward", "moe_backward_workspace_bytes",
                          "moe_expert_backward_input", "moe_expert_backward", "moe_router_backward",
                          "moe_router_backward_workspace_bytes", "moe_layer_forward_noalloc",
                          "moe_status_string"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings():
    assert moe.moe_status_string(0) == "ok"
    assert moe.moe_status_string(3) == "workspace too small"
    assert moe.moe_status_string(99) == "unknown status"


@pytest.mark.parametrize("kw,expected", [
    (dict(E=250), B.MOE_ERR_INVALID_ARGUMENT),           # E % G != 0
    (dict(M=0), B.MOE_ERR_INVALID_ARGUMENT),
    (dict(M=9), B.MOE_ERR_INVALID_ARGUMENT),             # M > G
    (dict(K=129, M=4), B.MOE_ERR_INVALID_ARGUMENT),      # K > M * E / G
    (dict(topn=33), B.MOE_ERR_INVALID_ARGUMENT),         # group_topn > E / G
    (dict(topn=0), B.MOE_ERR_INVALID_ARGUMENT),
    (dict(T=0), B.MOE_ERR_INVALID_ARGUMENT),
    (dict(Ns=-1), B.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=512, G=8), B.MOE_ERR_UNSUPPORTED),           # > 256 experts
    (dict(K=9), B.MOE_ERR_UNSUPPORTED),                  # > 8 per token
    (dict(topn=9), B.MOE_ERR_UNSUPPORTED),
    (dict(w="e4m3", hidden=7000), B.MOE_ERR_UNSUPPORTED),  # FP8 needs 128-multiples
    (dict(w="e4m3", inter=2000), B.MOE_ERR_UNSUPPORTED),
    (dict(w="e4m3_pow2", hidden=7000), B.MOE_ERR_UNSUPPORTED),
    (dict(act="e4m3_pow2", w="e4m3_pow2"), B.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", w="bf16"), B.MOE_ERR_UNSUPPORTED),  # dtype combination
    (dict(act="e4m3", w="e4m3"), B.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", w="f32", hidden=258), B.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs(kw, expected):
    c = cfg(**kw)
    assert moe.moe_workspace_bytes(c) == 0
    got = code_of(B.moe_route, c, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1 << 40,
                  stream=0)
    assert got == expected


def test_valid_configs_have_workspace():
    for kw in [dict(), dict(T=128), dict(w="e4m3"), dict(w="e4m3_pow2"), dict(T=16384),
               dict(T=64, hidden=256, inter=128, E=16, K=4, G=4, M=2, act="f32", w="f32")]:
        c = cfg(**kw)
        n = moe.moe_workspace_bytes(c)
        assert n > 0 and n % 256 == 0
    # y_rows and h (T*(K+Ns) rows each) dominate; FP8 adds one-byte codes of x and h
    assert moe.moe_workspace_bytes(cfg()) < moe.moe_workspace_bytes(cfg(w="e4m3")) < 2 * 10 ** 9
    assert moe.moe_workspace_bytes(cfg(w="e4m3")) == moe.moe_workspace_bytes(cfg(w="e4m3_pow2"))


def test_largest_token_count():
    # the MFMA kernels address h through 32-bit buffer offsets: 2 * T*(K+Ns) * inter bytes
    # must not exceed 2^31 - 2^20, so T = 58225 is the largest bf16 batch at this shape
    lim = (1 << 31) - (1 << 20)
    t_max = lim // (2 * 9 * 2048)
    assert t_max == 58225
    for w in ("bf16", "e4m3", "e4m3_pow2"):
        assert moe.moe_workspace_bytes(cfg(T=t_max, w=w)) > 0
        assert moe.moe_workspace_bytes(cfg(T=t_max + 1, w=w)) == 0
        got = code_of(B.moe_route, cfg(T=t_max + 1, w=w), ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                      ALIGNED, ALIGNED, 1 << 40, stream=0)
        assert got == B.MOE_ERR_UNSUPPORTED


def test_null_pointers_and_workspace_checks():
    c = cfg()
    need = moe.moe_workspace_bytes(c)
    A = ALIGNED
    assert code_of(B.moe_route, c, 0, A, A, A, A, A, need, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_route, c, A, A, A, A, A, A, need - 1, stream=0) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert code_of(B.moe_route, c, A, A, A, A, A, A + 16, need, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT                             # misaligned workspace
    assert code_of(B.moe_route, c, A, A, A, A, A, 0, need, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_permute, c, A, 0, A, A, A, A, need, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_permute, c, A, A, A, A, A, A, 0, stream=0) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert code_of(B.moe_combine, c, A, A, 0, None, A, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_bias_update, c, A, -1.0, A, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_bias_update, c, A, float("nan"), A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_bias_update, c, A, float("inf"), A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_bias_update, c, 0, 1e-3, A, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_act_quant_e4m3, c, A, 4, 100, A, A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT                             # cols not a multiple of 128
    assert code_of(B.moe_act_quant_e4m3, cfg(act="f32", w="f32"), A, 4, 128, A, A, stream=0) == \
        B.MOE_ERR_UNSUPPORTED


def test_balance_loss_argument_checks():
    c = cfg()
    need = moe.moe_workspace_bytes(c)
    A = ALIGNED

    def loss(seq_len=4096, alpha=1e-4, scores=A, idx=A, out=A, ws_bytes=need, ws=A):
        return code_of(B.moe_balance_loss, c, scores, idx, seq_len, alpha, out, None, None, None,
                       ws, ws_bytes, stream=0)

    assert loss(seq_len=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(seq_len=-8) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(seq_len=3000) == B.MOE_ERR_INVALID_ARGUMENT      # does not divide T = 8192
    assert loss(seq_len=16384) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(alpha=-1e-4) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(alpha=float("nan")) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(alpha=float("inf")) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(scores=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(idx=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(out=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert loss(ws_bytes=need - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert loss(ws=A + 64) == B.MOE_ERR_INVALID_ARGUMENT          # misaligned workspace
    assert code_of(B.moe_balance_loss, cfg(E=250), A, A, 10, 1e-4, A, None, None, None, A, need,
                   stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_router_scores, c, A, A, 0, A, need, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_router_scores, c, 0, A, A, A, need, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_router_scores, c, A, A, A, A, need - 1, stream=0) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL


def test_backward_argument_checks():
    c = cfg()
    A = ALIGNED
    args = [A] * 6
    for i in range(6):
        bad = list(args)
        bad[i] = 0
        assert code_of(B.moe_combine_backward, c, *bad, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    for i in range(4):
        bad = [A] * 4
        bad[i] = 0
        assert code_of(B.moe_gate_backward, c, *bad, stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_gate_backward, cfg(E=250), A, A, A, A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_combine_backward, cfg(act="f32", w="bf16"), *args, stream=0) == \
        B.MOE_ERR_UNSUPPORTED
    for i in range(5):
        bad = [A] * 5
        bad[i] = 0
        assert code_of(B.moe_swiglu_backward, c, bad[0], bad[1], bad[2], 16, bad[3], bad[4],
                       stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_swiglu_backward, c, A, A, A, 0, A, A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT


def test_expert_backward_argument_checks():
    A = ALIGNED
    c = cfg()
    need = moe.moe_backward_workspace_bytes(c)
    # row-sized buffers (a | b, dh, da | db, dX: 5 inter + hidden bf16 values per grouped
    # row) and the weight gradients' packed operands; nothing weight-sized
    rows = 8192 * 9
    assert rows * (5 * 2048 + 7168) * 2 < need < 257 * 3 * 7168 * 2048 * 2 and need % 256 == 0
    assert moe.moe_backward_workspace_bytes(cfg(w="e4m3")) == 0          # bf16 only
    assert moe.moe_backward_workspace_bytes(cfg(act="f32", w="f32", hidden=256, inter=128,
                                                T=64, E=16, K=4, G=4, M=2)) == 0
    assert moe.moe_backward_workspace_bytes(cfg(T=16635)) > 0            # rows * hidden * 2 limit
    assert moe.moe_backward_workspace_bytes(cfg(T=16636)) == 0
    dense = dict(w_gate=A, w_up=A, w_down=A)

    def call(conf=c, ws_bytes=need, ws=A, **kw):
        args = dict(x=A, off=A, rt=A, pr=A, w=dense, dy=A, dx=A)
        args.update(kw)
        return code_of(B.moe_expert_backward_input, conf, args["x"], args["off"], args["rt"],
                       args["pr"], args["w"], args["dy"], args["dx"], ws, ws_bytes, stream=0)

    for k in ("x", "off", "rt", "pr", "dy", "dx"):
        assert call(**{k: 0}) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(w=dict(dense, w_up=0)) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(w=dict(dense, s_gate=A, s_up=A, s_down=A)) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=need - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=A + 32) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(conf=cfg(w="e4m3")) == B.MOE_ERR_UNSUPPORTED

    def full(dx=A, dw=(A, A, A)):
        return code_of(B.moe_expert_backward, c, A, A, A, A, dense, A, dx, *dw, A, need,
                       stream=0)

    assert full(dx=0, dw=(0, 0, 0)) == B.MOE_ERR_INVALID_ARGUMENT       # nothing requested
    assert full(dw=(A, 0, A)) == B.MOE_ERR_INVALID_ARGUMENT             # all or none
    assert full(dw=(0, 0, A)) == B.MOE_ERR_INVALID_ARGUMENT
    rb = B.moe_router_backward
    rneed = moe.moe_router_backward_workspace_bytes(c)
    # hi | lo of the logit gradient twice (8192 x 512 bf16 each), W_r^T twice, x^T,
    # four split-K partials of [512, 7168] fp32
    assert rneed == 2 * 8192 * 512 * 2 + 7168 * 512 * 2 + 7168 * 8192 * 2 + 4 * 512 * 7168 * 4
    assert moe.moe_router_backward_workspace_bytes(cfg(act="f32", w="f32")) == 0
    assert moe.moe_router_backward_workspace_bytes(cfg(hidden=7164)) == 0
    assert moe.moe_router_backward_workspace_bytes(cfg(E=250, G=10, M=4)) > 0   # E padded to 256

    def router(conf=c, ws=A, ws_bytes=rneed, x=A, w=A, g=A, dx=A, dw=A):
        return code_of(rb, conf, x, w, g, dx, dw, ws, ws_bytes, stream=0)

    assert router(dx=0, dw=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert router(x=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert router(g=0, dw=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert router(ws=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert router(ws=A + 32) == B.MOE_ERR_INVALID_ARGUMENT
    assert router(ws_bytes=rneed - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert router(conf=cfg(act="f32", w="f32", hidden=256, inter=128, T=64, E=16, K=4, G=4,
                           M=2)) == B.MOE_ERR_UNSUPPORTED


def test_weight_scale_pointer_rules():
    A = ALIGNED
    need8 = moe.moe_workspace_bytes(cfg(w="e4m3"))
    dense = dict(w_gate=A, w_up=A, w_down=A)
    scaled = dict(dense, s_gate=A, s_up=A, s_down=A)
    # bf16 weights must not carry scales; e4m3 weights must
    assert code_of(B.moe_grouped_ffn, cfg(), A, A, A, scaled, A, A, need8, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_grouped_ffn, cfg(w="e4m3"), A, A, A, dense, A, A, need8, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_grouped_ffn, cfg(w="e4m3_pow2"), A, A, A, dense, A, A, need8,
                   stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_grouped_ffn, cfg(w="e4m3_pow2"), A, A, A, dict(scaled, s_up=0), A, A, need8,
                   stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_grouped_ffn, cfg(), A, A, A, dict(dense, w_up=0), A, A, need8,
                   stream=0) == B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(B.moe_layer_forward, cfg(), A, A, A, dense, None, A, A, A, 0, A, need8,
                   stream=0) == B.MOE_ERR_INVALID_ARGUMENT


def test_noalloc_argument_checks():
    """moe_layer_forward_noalloc rejects null pointers and batches whose workspace is
    beyond its 64 MiB array on the host, before it touches a device."""
    A = ALIGNED
    dense = dict(w_gate=A, w_up=A, w_down=A)
    fn = B.moe_layer_forward_noalloc
    assert moe.moe_workspace_bytes(cfg(T=365)) <= 64 << 20 < moe.moe_workspace_bytes(cfg(T=366))
    assert code_of(fn, cfg(T=366), A, A, A, dense, None, A, A, A, A, stream=0) == \
        B.MOE_ERR_UNSUPPORTED
    assert code_of(fn, cfg(), A, A, A, dense, None, A, A, A, A, stream=0) == B.MOE_ERR_UNSUPPORTED
    assert code_of(fn, cfg(T=128), 0, A, A, dense, None, A, A, A, A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(fn, cfg(T=128), A, A, A, dense, None, A, A, A, 0, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert code_of(fn, cfg(T=128, w="e4m3"), A, A, A, dense, None, A, A, A, A, stream=0) == \
        B.MOE_ERR_INVALID_ARGUMENT                             # scales missing
    assert code_of(fn, cfg(T=128, K=9), A, A, A, dense, None, A, A, A, A, stream=0) == \
        B.MOE_ERR_UNSUPPORTED


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        B.moe_bias_update(cfg(), torch.zeros(256, dtype=torch.int32), 1e-3,
                          torch.zeros(256), stream=0)


def test_config_struct_layout():
    # 9 int32 fields followed by two C enums (int): 44 bytes, no padding
    assert ctypes.sizeof(B.MoeConfig) == 44
    assert ctypes.sizeof(B.MoeExpertWeights) == 6 * ctypes.sizeof(ctypes.c_void_p)
