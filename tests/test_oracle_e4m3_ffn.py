"""Pins for the e4m3 format, the 1x128 / 128x128 FP8 block quantisation and the
SwiGLU expert / layer combination of the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float64).numpy()
    tab = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert nan.tolist() == np.isnan(tab).tolist()
    assert np.nonzero(nan)[0].tolist() == [0x7F, 0xFF]
    np.testing.assert_array_equal(tab[~nan], ref[~nan])
    assert np.nanmax(tab) == 448.0 and tab[0x01] == 2.0 ** -9


def test_e4m3_rne_matches_torch_cast_sweep():
    rng = np.random.default_rng(0)
    tab = oracle.e4m3_table()
    mids = (tab[1:0x7F] + tab[0:0x7E]) / 2           # every midpoint: the ties
    v = np.concatenate([
        rng.uniform(-448, 448, 200000), rng.standard_normal(100000) * 1e-2,
        mids, -mids, tab[:0x7F], np.nextafter(mids, 0), np.nextafter(mids, 1000),
        [0.0, -0.0, 447.99, -447.99, 2.0 ** -10, -(2.0 ** -11)],
    ]).astype(np.float32)
    ours = oracle.e4m3_encode_rne(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturates():
    v = np.array([448.0, 464.0, 1e6, -500.0, np.inf, -np.inf], np.float32)
    assert oracle.e4m3_encode_rne(v).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_quant_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals, scale, codes = (p.strip() for p in line.split("|"))
            rows.append(([float(v) for v in vals.split()], float(scale),
                         [int(c, 16) for c in codes.split()]))
    return rows


def test_quantize_1x128_golden():
    for vals, scale, codes in _golden_rows():
        x = np.zeros((1, 128), np.float32)
        x[0, :len(vals)] = vals
        q, s = oracle.quantize_1x128(x)
        assert s.shape == (1, 1) and s[0, 0] == np.float32(scale)
        assert q[0, :len(codes)].tolist() == codes
        assert np.all(q[0, len(codes):] == 0)


def test_quantize_1x128_bounds():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((16, 512)) * rng.uniform(0.01, 10, (16, 1))).astype(np.float32)
    x[3, 128:256] = 0.0
    q, s = oracle.quantize_1x128(x)
    assert s.shape == (16, 4) and s.dtype == np.float32 and s[3, 1] == 1.0
    tab = oracle.e4m3_table()
    deq = oracle.dequantize_1x128(q, s)
    blocks = x.reshape(16, 4, 128)
    amax = np.abs(blocks).max(2)
    # the block maximum maps to 448 (the largest code)
    for r in range(16):
        for j in range(4):
            if amax[r, j] > 0:
                k = np.argmax(np.abs(blocks[r, j]))
                assert abs(tab[q[r, j * 128 + k]]) == 448.0
    # error bound: at most half an e4m3 step (relative 2^-4) of each value, in scale units
    err = np.abs(deq - x) / np.repeat(s, 128, axis=1)
    step = np.abs(tab[q]) * 2.0 ** -3
    assert np.all(err <= np.maximum(step, 2.0 ** -9) / 2 * (1 + 1e-6) + 1e-12)


def test_dequantize_blocks_128():
    codes = torch.tensor([[0x38] * 256] * 256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    scales = np.array([[1.0, 2.0], [3.0, 4.0]], np.float32)
    w = oracle.dequantize_blocks_128(codes, scales)
    assert w.shape == (256, 256)
    assert w[0, 0] == 1.0 and w[0, 200] == 2.0 and w[200, 0] == 3.0 and w[255, 255] == 4.0


def _loops_ffn(u, wg, wu, wd):
    n, h = u.shape
    inter = wg.shape[0]
    out = np.zeros((n, h))
    for r in range(n):
        hid = []
        for i in range(inter):
            a = sum(u[r, c] * wg[i, c] for c in range(h))
            b = sum(u[r, c] * wu[i, c] for c in range(h))
            hid.append(a / (1 + np.exp(-a)) * b)
        for c in range(h):
            out[r, c] = sum(hid[i] * wd[c, i] for i in range(inter))
    return out


def test_expert_ffn_matches_loops():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((3, 5))
    wg, wu, wd = rng.standard_normal((4, 5)), rng.standard_normal((4, 5)), rng.standard_normal((5, 4))
    np.testing.assert_allclose(oracle.expert_ffn(u, wg, wu, wd), _loops_ffn(u, wg, wu, wd),
                               rtol=1e-12, atol=1e-12)
    assert np.all(oracle.expert_ffn(u, wg, np.zeros_like(wu), wd) == 0)
    # silu closed form at a few points
    a = np.array([-3.0, 0.0, 0.5, 10.0])
    np.testing.assert_allclose(oracle.silu(a), a * (1 / (1 + np.exp(-a))), rtol=1e-15)


def _experts(rng, n, h, inter):
    return [(rng.standard_normal((inter, h)) * 0.3, rng.standard_normal((inter, h)) * 0.3,
             rng.standard_normal((h, inter)) * 0.3) for _ in range(n)]


def test_layer_one_hot_and_dense_mixture():
    rng = np.random.default_rng(3)
    E, h, inter, T = 8, 6, 5, 7
    ex = _experts(rng, E + 1, h, inter)
    x = rng.standard_normal((T, h))
    w = rng.standard_normal((E, h))
    # K = 1: the single gate is exactly 1 -> shared + the chosen expert
    r = oracle.route(x, w, np.zeros(E, np.float32), 1, 1, 1, 1)
    assert np.all(r.gate == 1.0)
    y = oracle.layer_output(x, r.idx, r.gate, lambda e: ex[e], E, 1)
    for t in range(T):
        ref = oracle.expert_ffn(x[t:t + 1], *ex[E]) + oracle.expert_ffn(x[t:t + 1], *ex[r.idx[t, 0]])
        np.testing.assert_allclose(y[t:t + 1], ref, rtol=1e-12)
    # M = G and K = E: a dense mixture weighted by s / sum(s) over all experts
    r = oracle.route(x, w, np.zeros(E, np.float32), 2, 2, 2, E)
    y = oracle.layer_output(x, r.idx, r.gate, lambda e: ex[e], E, 1)
    s = 1 / (1 + np.exp(-(x @ w.T)))
    ref = oracle.expert_ffn(x, *ex[E])
    for e in range(E):
        ref = ref + (s[:, e] / s.sum(1))[:, None] * oracle.expert_ffn(x, *ex[e])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # residual adds u; a subset of rows equals the same rows of the full output
    y_res = oracle.layer_output(x, r.idx, r.gate, lambda e: ex[e], E, 1, residual=x)
    np.testing.assert_allclose(y_res - x, y, rtol=1e-12, atol=1e-12)
    ys = oracle.layer_output(x, r.idx, r.gate, lambda e: ex[e], E, 1, rows=[1, 4])
    np.testing.assert_allclose(ys, y[[1, 4]], rtol=1e-15, atol=0)


def test_fp8_emulated_close_to_exact():
    rng = np.random.default_rng(4)
    h, inter = 256, 128
    u = rng.standard_normal((8, h)).astype(np.float32)
    wg, wu, wd = (rng.standard_normal((inter, h)) * 0.05, rng.standard_normal((inter, h)) * 0.05,
                  rng.standard_normal((h, inter)) * 0.05)
    exact = oracle.expert_ffn(u, wg, wu, wd)
    emu = oracle.expert_ffn_fp8_emulated(u, wg, wu, wd)
    rel = np.abs(emu - exact).max() / np.abs(exact).max()
    assert 1e-4 < rel < 0.1


def _pow2_brute(a: float) -> float:
    """The smallest 2^k (integer k >= -126) with a <= 448 * 2^k, found by scanning k."""
    if a == 0.0:
        return 1.0
    for k in range(-126, 140):
        if a <= 448.0 * 2.0 ** k:
            return 2.0 ** k
    raise AssertionError(a)


def test_pow2_scale_hand_values_and_brute_force():
    # hand values: 448 = 448 * 2^0; 449 needs 2^1; 1 <= 448 * 2^-8 = 1.75 but > 0.875
    assert oracle.pow2_scale([448.0, 449.0, 1.0, 224.0, 0.0]).tolist() == [1.0, 2.0, 2.0 ** -8, 0.5, 1.0]
    assert oracle.pow2_scale([1e-40, 448.0 * 2.0 ** -126, 448.0 * 2.0 ** -125]).tolist() == \
        [2.0 ** -126, 2.0 ** -126, 2.0 ** -125]
    rng = np.random.default_rng(11)
    a = np.concatenate([
        np.exp(rng.uniform(-40, 40, 3000)).astype(np.float32),
        np.float32(448.0) * np.ldexp(np.float32(1.0), rng.integers(-30, 30, 200)).astype(np.float32),
        np.nextafter(np.float32(448.0) * np.ldexp(np.float32(1.0), rng.integers(-30, 30, 200)).astype(np.float32),
                     np.float32(np.inf)),
    ]).astype(np.float32)
    s = oracle.pow2_scale(a)
    assert s.dtype == np.float32
    for ai, si in zip(a.tolist(), s.tolist()):
        assert si == _pow2_brute(ai), (ai, si)
    m, _ = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)                                  # powers of two
    assert np.all(a <= 448.0 * s.astype(np.float64)) and np.all(a > 224.0 * s.astype(np.float64))


def test_quantize_1x128_pow2_exact_and_bounded():
    rng = np.random.default_rng(12)
    tab = oracle.e4m3_table()
    # blocks made of e4m3 values times a power of two quantise exactly when the block
    # amax is a power-of-two multiple of 448 (then the scale is that power)
    codes = rng.integers(0, 0x7E, (4, 256)).astype(np.uint8) | (rng.integers(0, 2, (4, 256)) * 0x80).astype(np.uint8)
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    p = np.ldexp(1.0, rng.integers(-10, 10, (4, 2)))
    x = (tab[codes].reshape(4, 2, 128) * p[:, :, None]).reshape(4, 256).astype(np.float32)
    q, s = oracle.quantize_1x128_pow2(x)
    assert np.array_equal(s.astype(np.float64), p)
    assert np.array_equal(q, codes)
    # random data: power-of-two scales, the half-step bound, magnitudes <= 448
    x = (rng.standard_normal((16, 512)) * rng.uniform(0.01, 10, (16, 1))).astype(np.float32)
    x[5, :128] = 0.0
    q, s = oracle.quantize_1x128_pow2(x)
    assert s[5, 0] == 1.0 and np.all(q[5, :128] == 0)
    m, _ = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)
    deq = oracle.dequantize_1x128(q, s)
    err = np.abs(deq - x) / np.repeat(s, 128, axis=1)
    step = np.abs(tab[q]) * 2.0 ** -3
    assert np.all(np.abs(tab[q]) <= 448.0)
    assert np.all(err <= np.maximum(step, 2.0 ** -9) / 2 * (1 + 1e-6) + 1e-12)
    # differs from the amax / 448 rule: the block maximum usually no longer maps to 448
    q2, _ = oracle.quantize_1x128(x)
    assert not np.array_equal(q, q2)


def test_fp8_pow2_emulated_close_to_exact():
    rng = np.random.default_rng(13)
    h, inter = 256, 128
    u = rng.standard_normal((8, h)).astype(np.float32)
    wg, wu, wd = (rng.standard_normal((inter, h)) * 0.05, rng.standard_normal((inter, h)) * 0.05,
                  rng.standard_normal((h, inter)) * 0.05)
    exact = oracle.expert_ffn(u, wg, wu, wd)
    emu = oracle.expert_ffn_fp8_pow2_emulated(u, wg, wu, wd)
    rel = np.abs(emu - exact).max() / np.abs(exact).max()
    assert 1e-4 < rel < 0.1
    assert not np.array_equal(emu, oracle.expert_ffn_fp8_emulated(u, wg, wu, wd))


# ---- hand-worked FP8 expert (devpress page, section 2: 1x128 activation tiles) ------
# One token, hidden = inter = 256: two 128-wide K blocks in each GEMM, so each tile's
# own scale matters.  Every value below is derived by hand (the derivation is in the
# comments); the oracle must reproduce them exactly.
#
# x, block 0: x0 = 14 is the block maximum, so s = 14 / 448 = 2^-5 (exact) and the
#   quotients are x / 2^-5: 14 -> 448 (exact), 0.08 -> 2.56 -> e4m3 2.5 (grid 0.25 on
#   [2, 4)), 0.3 -> 9.6 -> 10 (grid 1 on [8, 16)).  Dequantised: 14, 0.078125, 0.3125.
# x, block 1: x128 = 0.875 is the maximum, s = 0.875 / 448 = 2^-9 (exact):
#   0.0107 -> 5.4784 -> 5.5 (grid 0.5 on [4, 8)) -> 0.0107421875;
#   0.00035 -> 0.1792 -> 0.171875 (grid 2^-6 on [1/8, 1/4)) -> 11 / 32768.
#   With one scale per row (2^-5) instead, 0.00035 -> 0.0112, subnormal (grid 2^-9):
#   -> 6 * 2^-9 -> 12 / 32768: a per-row scale changes the result.
# Gate rows read x0 with weight 4: a = 56 and silu(56) = 56 in float64
#   (56 / (1 + e^-56), e^-56 ~ 5e-25 is below half an ulp).
# Up rows: b0 = xq1 = 0.078125, b1 = xq2 = 0.3125, b2 = 0.0301 * xq0 = 0.4214,
#   b128 = 2^16 * xq130 = 22, b129 = 2^10 * xq129 = 11.
# h = 56 b: 4.375, 17.5, 23.5984 (float64), 1232, 616; in bf16 (7 stored bits)
#   23.5984 -> 23.625 (grid 0.125 on [16, 32)); the others are exact.
# h, block 0: s = 23.625 / 448 = 27 / 512 (exact); quotients 4.375 * 512/27 = 82.96 -> 80
#   (grid 8 on [64, 128)), 17.5 * 512/27 = 331.85 -> 320 (grid 32 on [256, 512)), 448.
#   Dequantised: 80 * 27/512 = 4.21875, 320 * 27/512 = 16.875, 23.625.
# h, block 1: s = 1232 / 448 = 2.75, quotients 448 and 616 / 2.75 = 224 (exact).
# W_down copies h columns 0, 1, 2, 128, 129 to outputs 0..4 and sends
#   h0 + 2 h128 to output 5 (a sum over both K blocks of GEMM2).
_HAND_Y = [4.21875, 16.875, 23.625, 1232.0, 616.0, 4.21875 + 2 * 1232.0]
# power-of-two scales (the smallest 2^k with amax <= 448 * 2^k): x keeps 2^-5 and 2^-9
# (its maxima are 448 times a power of two), so xq is unchanged; h block 0: 23.625 <=
# 448 * 2^-4, s = 1/16: 4.375 -> 70 -> 72 (grid 8) -> 4.5; 17.5 -> 280 -> 288 (grid
# 32) -> 18; 23.625 -> 378 -> 384 -> 24.  h block 1: 1232 <= 448 * 4, s = 4: 1232 ->
# 308 -> 320 -> 1280; 616 -> 154 -> 160 (grid 16 on [128, 256)) -> 640.
_HAND_Y_POW2 = [4.5, 18.0, 24.0, 1280.0, 640.0, 4.5 + 2 * 1280.0]


def _hand_expert():
    x = np.zeros((1, 256), np.float32)
    x[0, [0, 1, 2, 128, 129, 130]] = [14.0, 0.08, 0.3, 0.875, 0.0107, 0.00035]
    wg = np.zeros((256, 256))
    wu = np.zeros((256, 256))
    wd = np.zeros((256, 256))
    wg[[0, 1, 2, 128, 129], 0] = 4.0
    wu[0, 1] = 1.0
    wu[1, 2] = 1.0
    wu[2, 0] = 0.0301
    wu[128, 130] = 2.0 ** 16
    wu[129, 129] = 2.0 ** 10
    for c, i in enumerate([0, 1, 2, 128, 129]):
        wd[c, i] = 1.0
    wd[5, 0] = 1.0
    wd[5, 128] = 2.0
    return x, wg, wu, wd


def _quant_per_row(v):
    """A planted mistake: one scale per row instead of one per 1x128 tile."""
    v = np.asarray(v, np.float32)
    s = (np.abs(v).max(1, keepdims=True) / np.float32(448)).astype(np.float32)
    return oracle.e4m3_table()[oracle.e4m3_encode_rne((v / s).astype(np.float32))] * s.astype(np.float64)


def _variant(x, wg, wu, wd, quant_x=True, quant_h=True, bf16_h=True, pow2=False, row_x=False,
             row_h=False, swap=False):
    """The FP8-emulating expert with one step switched (a planted mistake each)."""
    quant = oracle.quantize_1x128_pow2 if pow2 else oracle.quantize_1x128
    tile = lambda v: oracle.dequantize_1x128(*quant(v))
    xq = (_quant_per_row(x) if row_x else tile(x)) if quant_x else np.asarray(x, np.float64)
    a, b = xq @ wg.T, xq @ wu.T
    h = oracle.silu(b) * a if swap else oracle.silu(a) * b
    hb = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).float().numpy() if bf16_h \
        else h.astype(np.float32)
    hq = (_quant_per_row(hb) if row_h else tile(hb)) if quant_h else h
    return hq @ wd.T


def test_fp8_emulated_hand_case():
    x, wg, wu, wd = _hand_expert()
    y = oracle.expert_ffn_fp8_emulated(x, wg, wu, wd)
    assert y[0, :6].tolist() == _HAND_Y and np.all(y[0, 6:] == 0)
    # the unswitched variant is the same computation
    assert np.array_equal(_variant(x, wg, wu, wd), y)
    # each planted mistake moves at least one hand-derived output
    for mistake in (dict(quant_h=False), dict(quant_x=False), dict(bf16_h=False), dict(pow2=True),
                    dict(row_x=True), dict(row_h=True), dict(swap=True)):
        got = _variant(x, wg, wu, wd, **mistake)[0, :6]
        assert np.abs(got - np.array(_HAND_Y)).max() > 1e-3, mistake


def test_fp8_pow2_emulated_hand_case():
    x, wg, wu, wd = _hand_expert()
    y = oracle.expert_ffn_fp8_pow2_emulated(x, wg, wu, wd)
    assert y[0, :6].tolist() == _HAND_Y_POW2 and np.all(y[0, 6:] == 0)
    assert np.array_equal(_variant(x, wg, wu, wd, pow2=True), y)
    for mistake in (dict(quant_h=False), dict(quant_x=False), dict(pow2=False),
                    dict(swap=True)):
        got = _variant(x, wg, wu, wd, **{"pow2": True, **mistake})[0, :6]
        assert np.abs(got - np.array(_HAND_Y_POW2)).max() > 1e-3, mistake
