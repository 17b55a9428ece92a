"""OCP FP8 E4M3 (e4m3fn) encoding and the blockwise FP8 expert path (test infrastructure only).

Sources (the pages):
  * "DeepSeek-V3 ... 技术解析" (devpress), section 2: weights are quantised per 128x128
    block and activations per 1x128 tile; heavy matmuls run in FP8 with FP32
    accumulation every 128 elements.
  * stapisi blog, section 6.2: the largest E4M3 value is 448.

Format (OCP 8-bit floating point, E4M3 "fn" variant): sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); no infinities;
S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448.

Readings (listed in the design notes):
  * block scale s = amax / 448 as a float32 division, s = 1 when amax == 0
  * code = round-to-nearest-even of the float32 quotient x / s, saturating at +-448;
    the sign of a value that rounds to zero is kept (0x80 for negative values)
  * a quantised GEMM equals sum over 128-wide K blocks of (s_a * s_w * sum q_a q_w);
    the oracle computes it as the exact product of dequantised values.
  * power-of-two variant (scales an 8-bit exponent, E8M0, can hold; the pages give the
    block shapes, not the scale encoding): s = the smallest power of two with
    amax <= 448 * s, at least 2^-126 (1 when amax == 0); codes as above, the quotient
    x / s being exact.
    Weight block scales of this variant are powers of two as stored.
"""
from __future__ import annotations

import numpy as np

from .moe_layer import _f64, silu

E4M3_MAX = 448.0


def e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3fn codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_POS = e4m3_table()[:0x7F]          # codes 0x00..0x7E: 0, ..., 448, ascending


def e4m3_encode_rne(v) -> np.ndarray:
    """Round values to e4m3 codes: nearest, ties to the even code, saturate at +-448.

    Works on the exact float64 value of the input (float32 inputs are exact in float64).
    NaN maps to 0x7F.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    lo = np.clip(np.searchsorted(_POS, a, side="right") - 1, 0, 0x7E)   # _POS[lo] <= a
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def quantize_1x128(x):
    """Per row and per 128-column block: s = f32(amax / 448) (1 if amax == 0),
    code = e4m3_rne(f32(x / s)).  x [rows, cols] with cols % 128 == 0 (float32-exact values).

    Returns (codes uint8 [rows, cols], scales float32 [rows, cols/128]).
    """
    x32 = np.asarray(_f64(x), dtype=np.float32)
    rows, cols = x32.shape
    blocks = x32.reshape(rows, cols // 128, 128)
    amax = np.abs(blocks).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quot = (blocks / scale[:, :, None]).astype(np.float32)
    return e4m3_encode_rne(quot).reshape(rows, cols), scale


def pow2_scale(amax) -> np.ndarray:
    """Smallest power of two s >= 2^-126 with amax <= 448 s (s = 1 for amax == 0), exact.

    With amax = m 2^E, m in [0.5, 1): 448 = 0.875 2^9, so s = 2^(E-9) when m <= 0.875 and
    2^(E-8) otherwise.  The floor 2^-126 keeps s a normal float32 (its exponent field
    is then its 8-bit exponent code).  Returned as float32."""
    a = np.asarray(amax, np.float64)
    m, e = np.frexp(a)
    s = np.ldexp(1.0, np.maximum(np.where(m <= 0.875, e - 9, e - 8), -126))
    return np.where(a > 0, s, 1.0).astype(np.float32)


def quantize_1x128_pow2(x):
    """quantize_1x128 with power-of-two block scales (pow2_scale of the block amax)."""
    x32 = np.asarray(_f64(x), dtype=np.float32)
    rows, cols = x32.shape
    blocks = x32.reshape(rows, cols // 128, 128)
    scale = pow2_scale(np.abs(blocks).max(axis=2))
    quot = blocks.astype(np.float64) / scale[:, :, None].astype(np.float64)   # exact
    return e4m3_encode_rne(quot).reshape(rows, cols), scale


def dequantize_1x128(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    vals = e4m3_table()[codes].reshape(rows, cols // 128, 128)
    return (vals * np.asarray(scales, np.float64)[:, :, None]).reshape(rows, cols)


def dequantize_blocks_128(codes, scales) -> np.ndarray:
    """Weights stored as e4m3 codes [n, k] with one scale per 128x128 block [n/128, k/128]."""
    if hasattr(codes, "detach"):
        codes = codes.detach().to("cpu").view(__import__("torch").uint8).numpy()
    codes = np.asarray(codes, dtype=np.uint8)
    sc = _f64(scales)
    n, k = codes.shape
    vals = e4m3_table()[codes]
    return vals * np.repeat(np.repeat(sc, 128, axis=0), 128, axis=1)[:n, :k]


def _round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float32."""
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def expert_ffn_fp8_emulated(u, w_gate, w_up, w_down, pow2: bool = False) -> np.ndarray:
    """Diagnostic FP8 expert: u and the SwiGLU output h are each quantised per 1x128
    along their own K dimension before the GEMM that consumes them (power-of-two
    scales if pow2); weights are already dequantised float64 arrays.  Products and
    sums in float64.

    The pages fix no storage precision for h between the two GEMMs; the kernels
    hold it in bf16, so the FP8 codes of h are decided on the bf16-rounded value
    (a code is decided in the kernel's precision where the pages are silent)."""
    quant = quantize_1x128_pow2 if pow2 else quantize_1x128
    uq = dequantize_1x128(*quant(np.asarray(_f64(u), np.float32)))
    h = silu(uq @ _f64(w_gate).T) * (uq @ _f64(w_up).T)
    hq = dequantize_1x128(*quant(_round_bf16(h)))
    return hq @ _f64(w_down).T


def expert_ffn_fp8_pow2_emulated(u, w_gate, w_up, w_down) -> np.ndarray:
    """expert_ffn_fp8_emulated with power-of-two activation scales."""
    return expert_ffn_fp8_emulated(u, w_gate, w_up, w_down, pow2=True)
