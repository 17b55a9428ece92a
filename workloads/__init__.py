"""Seeded synthetic workloads for the DeepSeekMoE layer forward.

This module only *draws* inputs: shapes, value distributions and seeds.  It holds
none of the layer's arithmetic (no affinity, routing, permutation, FFN, combine,
bias update or quantisation), so both the CPU oracle and the HIP path can take
their inputs from it without sharing any of the method.

Workloads (the layer of the DeepSeek-V3 technical report summary, section 2.2
"DeepSeekMoE": 256 routed experts + 1 shared expert, 8 routed experts per token):

* ``tiny_fp32``    T=64,    h=256,  inter=128,  E=16,  K=4, G=4, M=2, fp32
* ``decode_bf16``  T=128,   h=7168, inter=2048, E=256, K=8, G=8, M=4, bf16,
                   bias ~ U(-0.01, 0.01)
* ``prefill_bf16`` T=8192,  same shapes, bf16, bias = 0
* ``prefill_fp8``  T=8192,  expert weights stored as OCP e4m3 codes with one fp32
                   scale per 128x128 block; activations bf16
* ``prefill_fp8_pow2`` the same with power-of-two block scales (each scale above
                   rounded down to a power of two: 2^-13 or 2^-12)
* ``skewed_bf16``  T=16384, 8 hot experts (router logit offset +2.0 on experts
                   0..7, realised as input channel 0 == 1.0 and W_r[e, 0] = 2.0
                   for hot experts, 0 otherwise), 50 steps with gamma = 1e-3

Distributions: x ~ N(0, 1); router and expert weights ~ N(0, 0.02^2); every
value is drawn in fp32 and cast (round-to-nearest-even) to its storage dtype.
FP8 weights are drawn directly in their stored form: codes are the e4m3 cast of
N(0, 100^2) values clipped to +-448, and each 128x128 block carries its own
scale 0.02/100 * U(0.5, 1.5), so a dequantised weight is roughly N(0, 0.02^2).

Every tensor has its own torch.Generator seeded from (workload seed, tensor
name, expert id, step), so any one expert can be regenerated alone and the draw
is reproducible on a given device type.  The same seed gives different numbers
on CPU and on GPU (different generator algorithms); a comparison always feeds
both sides the same materialised tensors.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import torch

__all__ = ["MoeShape", "WORKLOADS", "get", "make_layer_inputs", "make_tokens",
           "sample_rows", "tensor_seed"]


@dataclasses.dataclass(frozen=True)
class MoeShape:
    name: str
    T: int              # tokens
    hidden: int         # h
    inter: int          # SwiGLU intermediate size (routed and shared experts)
    E: int              # routed experts N_r
    K: int              # routed experts per token K_r
    G: int              # expert groups ("nodes")
    M: int              # groups kept per token
    topn: int           # experts summed into a group score
    Ns: int             # shared experts
    act: str            # "f32" | "bf16"   (x, router weight, output)
    w: str              # "f32" | "bf16" | "e4m3" | "e4m3_pow2"   (expert weights)
    bias: str           # "zero" | "uniform"
    bias_range: float = 0.0
    hot: int = 0        # number of hot experts (skewed workload)
    hot_offset: float = 0.0
    steps: int = 1
    gamma: float = 1e-3
    seed: int = 0
    compare_rows: Optional[int] = None   # None: all rows; else a seeded subset

    def replace(self, **kw) -> "MoeShape":
        return dataclasses.replace(self, **kw)

    @property
    def rows(self) -> int:
        """Rows of the grouped FFN: one per (token, routed expert) pair plus the shared rows."""
        return self.T * self.K + self.T * self.Ns


WORKLOADS: Dict[str, MoeShape] = {
    "tiny_fp32": MoeShape("tiny_fp32", T=64, hidden=256, inter=128, E=16, K=4, G=4, M=2,
                          topn=2, Ns=1, act="f32", w="f32", bias="zero"),
    "decode_bf16": MoeShape("decode_bf16", T=128, hidden=7168, inter=2048, E=256, K=8, G=8,
                            M=4, topn=2, Ns=1, act="bf16", w="bf16", bias="uniform",
                            bias_range=0.01),
    "prefill_bf16": MoeShape("prefill_bf16", T=8192, hidden=7168, inter=2048, E=256, K=8,
                             G=8, M=4, topn=2, Ns=1, act="bf16", w="bf16", bias="zero",
                             compare_rows=512),
    "prefill_fp8": MoeShape("prefill_fp8", T=8192, hidden=7168, inter=2048, E=256, K=8,
                            G=8, M=4, topn=2, Ns=1, act="bf16", w="e4m3", bias="zero",
                            compare_rows=512),
    "prefill_fp8_pow2": MoeShape("prefill_fp8_pow2", T=8192, hidden=7168, inter=2048, E=256,
                                 K=8, G=8, M=4, topn=2, Ns=1, act="bf16", w="e4m3_pow2",
                                 bias="zero", compare_rows=512),
    "skewed_bf16": MoeShape("skewed_bf16", T=16384, hidden=7168, inter=2048, E=256, K=8,
                            G=8, M=4, topn=2, Ns=1, act="bf16", w="bf16", bias="zero",
                            hot=8, hot_offset=2.0, steps=50, gamma=1e-3, compare_rows=512),
}

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn,
           "e4m3_pow2": torch.float8_e4m3fn}


def is_fp8(w: str) -> bool:
    """Expert weights stored as e4m3 codes with 128x128 block scales."""
    return w in ("e4m3", "e4m3_pow2")
FP8_CODE_STD = 100.0   # std of the values whose e4m3 cast gives the stored codes


def get(name: str) -> MoeShape:
    return WORKLOADS[name]


def tensor_seed(seed: int, name: str, expert: int = -1, step: int = 0) -> int:
    """Stable 63-bit seed for one tensor of one workload."""
    key = f"{seed}/{name}/{expert}/{step}".encode()
    return (zlib.crc32(key) << 31 ^ zlib.crc32(key[::-1])) & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, seed, device, dtype):
    g = _gen(device, seed)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def _uniform(shape, lo, hi, seed, device):
    g = _gen(device, seed)
    v = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return v.mul_(hi - lo).add_(lo)


def make_tokens(cfg: MoeShape, step: int = 0, device="cpu") -> torch.Tensor:
    """x [T, h] in the activation dtype; a fresh seeded batch per step."""
    x = _normal((cfg.T, cfg.hidden), 1.0, tensor_seed(cfg.seed, "x", -1, step), device,
                torch.float32)
    if cfg.hot:
        x[:, 0] = 1.0     # carries the hot-expert logit offset through W_r[:, 0]
    return x.to(_DTYPES[cfg.act])


def make_router(cfg: MoeShape, device="cpu") -> torch.Tensor:
    w = _normal((cfg.E, cfg.hidden), 0.02, tensor_seed(cfg.seed, "w_router"), device,
                torch.float32)
    if cfg.hot:
        w[:, 0] = 0.0
        w[:cfg.hot, 0] = cfg.hot_offset
    return w.to(_DTYPES[cfg.act])


def make_bias(cfg: MoeShape, device="cpu") -> torch.Tensor:
    if cfg.bias == "uniform":
        return _uniform((cfg.E,), -cfg.bias_range, cfg.bias_range,
                        tensor_seed(cfg.seed, "bias"), device)
    return torch.zeros(cfg.E, dtype=torch.float32, device=device)


def _expert_matrix(cfg: MoeShape, name: str, e: int, rows: int, cols: int, device):
    """One expert's weight matrix [rows, cols] in the stored form.

    Returns (values, scales): scales is None unless the weights are e4m3, in which
    case it is the fp32 block-scale grid [rows/128, cols/128].
    """
    seed = tensor_seed(cfg.seed, name, e)
    if not is_fp8(cfg.w):
        return _normal((rows, cols), 0.02, seed, device, _DTYPES[cfg.w]), None
    v = _normal((rows, cols), FP8_CODE_STD, seed, device, torch.float32)
    codes = v.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    s = _uniform((rows // 128, cols // 128), 0.5, 1.5, tensor_seed(cfg.seed, name + "/scale", e),
                 device).mul_(0.02 / FP8_CODE_STD)
    if cfg.w == "e4m3_pow2":          # stored scales are powers of two: 2^-13 or 2^-12
        s = torch.exp2(torch.floor(torch.log2(s)))
    return codes, s


def make_layer_inputs(cfg: MoeShape, device="cpu", step: int = 0) -> dict:
    """All inputs of one layer forward, materialised on ``device``.

    Expert tensors are stacked routed-first: experts 0..E-1 routed, E..E+Ns-1 shared.
    w_gate, w_up: [E+Ns, inter, h]; w_down: [E+Ns, h, inter]; e4m3 scales
    s_gate, s_up: [E+Ns, inter/128, h/128]; s_down: [E+Ns, h/128, inter/128].
    """
    n_exp = cfg.E + cfg.Ns
    wdt = _DTYPES[cfg.w]
    out = {
        "x": make_tokens(cfg, step, device),
        "w_router": make_router(cfg, device),
        "bias": make_bias(cfg, device),
        "w_gate": torch.empty((n_exp, cfg.inter, cfg.hidden), dtype=wdt, device=device),
        "w_up": torch.empty((n_exp, cfg.inter, cfg.hidden), dtype=wdt, device=device),
        "w_down": torch.empty((n_exp, cfg.hidden, cfg.inter), dtype=wdt, device=device),
    }
    if is_fp8(cfg.w):
        out["s_gate"] = torch.empty((n_exp, cfg.inter // 128, cfg.hidden // 128),
                                    dtype=torch.float32, device=device)
        out["s_up"] = torch.empty_like(out["s_gate"])
        out["s_down"] = torch.empty((n_exp, cfg.hidden // 128, cfg.inter // 128),
                                    dtype=torch.float32, device=device)
    for e in range(n_exp):
        for name, rows, cols in (("w_gate", cfg.inter, cfg.hidden), ("w_up", cfg.inter, cfg.hidden),
                                 ("w_down", cfg.hidden, cfg.inter)):
            vals, scales = _expert_matrix(cfg, name, e, rows, cols, device)
            out[name][e].copy_(vals)
            if scales is not None:
                out["s" + name[1:]][e].copy_(scales)
    return out


def sample_rows(T: int, n: int, seed: int = 0) -> torch.Tensor:
    """Seeded sorted subset of n distinct token indices out of T (all of them if n >= T)."""
    if n >= T:
        return torch.arange(T)
    g = _gen("cpu", tensor_seed(seed, "sample_rows", n, T))
    return torch.sort(torch.randperm(T, generator=g)[:n]).values


def make_topk_indices(T: int, E: int, K: int, hot: int = 0, hot_weight: float = 0.0,
                      seed: int = 0) -> torch.Tensor:
    """Seeded [T, K] int32 expert choices, K distinct per token (a permutation-stage input).

    With hot > 0 the first ``hot`` experts are favoured (their random keys are raised
    by hot_weight), which leaves many experts empty for small T.
    """
    g = _gen("cpu", tensor_seed(seed, "topk", T, E * 16 + K))
    keys = torch.rand((T, E), generator=g)
    if hot:
        keys[:, :hot] += hot_weight
    return torch.topk(keys, K, dim=1).indices.to(torch.int32)


def make_affinities(T: int, E: int, seed: int = 0) -> torch.Tensor:
    """Seeded [T, E] float32 affinities, uniform in (0.02, 0.98) (a balance-loss-stage
    input: any values a sigmoid can produce)."""
    return _uniform((T, E), 0.02, 0.98, tensor_seed(seed, "affinities", T, E), "cpu")


def make_dense(shape, dtype: str = "bf16", std: float = 1.0, seed: int = 0,
               name: str = "dense") -> torch.Tensor:
    """Seeded N(0, std^2) tensor of any shape, drawn in float32 and rounded to
    ``dtype`` (stand-in activations and output gradients for the backward stages)."""
    n = 1
    for d in shape:
        n *= int(d)
    return _normal(tuple(shape), std, tensor_seed(seed, name, n), "cpu", _DTYPES[dtype])


def make_gates(T: int, K: int, seed: int = 0) -> torch.Tensor:
    """Seeded [T, K] float32 gate-like weights, uniform in (0.05, 1)."""
    return _uniform((T, K), 0.05, 1.0, tensor_seed(seed, "gates", T, K), "cpu")


def make_loads(E: int, T: int, K: int, seed: int = 0, at_mean: int = 4) -> torch.Tensor:
    """Seeded per-expert loads summing to T*K, the first ``at_mean`` exactly at the mean
    when T*K is a multiple of E (a bias-update-stage input)."""
    g = _gen("cpu", tensor_seed(seed, "loads", E, T * K))
    idx = torch.randint(0, E, (T * K,), generator=g)
    load = torch.bincount(idx, minlength=E)
    at_mean = min(at_mean, E - 1)           # one expert must absorb the surplus
    if (T * K) % E == 0 and at_mean > 0:
        mean = T * K // E
        surplus = int((load[:at_mean] - mean).sum())
        load[:at_mean] = mean
        load[at_mean] += surplus              # keep the total
    return load.to(torch.int32)

def topk_with_loads(T: int, K: int, loads) -> torch.Tensor:
    """[T, K] int32 expert choices whose per-expert counts are exactly ``loads`` (each at
    most T, summing to T*K), K distinct experts per token: the choices listed expert by
    expert fill the slots column by column, so a token's K slots lie T apart in the list
    and never repeat an expert.  A permutation-stage input with a prescribed histogram
    (row-block edge cases of the grouped GEMMs)."""
    loads = [int(v) for v in loads]
    assert sum(loads) == T * K and max(loads) <= T
    flat = torch.cat([torch.full((n,), e, dtype=torch.int32) for e, n in enumerate(loads) if n])
    return flat.reshape(K, T).t().contiguous()
