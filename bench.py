#!/usr/bin/env python3
"""Benchmark of the MI355X DeepSeekMoE layer forward (one GPU).

One step = one pass of the whole hot path on one resident batch, through the
C ABI stage calls on one stream:
    moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine -> moe_bias_update
(the same kernels moe_layer_forward enqueues, plus the end-of-step bias update).
Inputs (x, router, bias, 257 experts' weights) are generated on the GPU before
timing.  W warm-up steps, then exactly K timed steps between two synchronisations;
HIP events recorded on the same stream time every stage of every timed step.

Prints ONE JSON line: layer tokens/s as ``value``, plus the grouped-GEMM TFLOP/s
and the roofline of the grouped expert GEMM (moe_grouped_ffn: the gated GEMM1 and
GEMM2 kernels, 99.5% of the layer's FLOPs) and the CPU oracle's rate on a bounded
sample (``cpu_baseline``).  After the timed steps, and outside them, the
training-side extras are timed on their own: the router affinities and the
sequence-wise balance loss with its logit gradient (``balance_loss``), and the
combine, gate and SwiGLU backward (``backward``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "e4m3": 5000.0, "e4m3_pow2": 5000.0, "f32": 157.3}   # dense TFLOP/s, MI355X
HBM_PEAK = 8000.0                                         # GB/s
METRIC = "MoE layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), T=8192 h=7168 E=256 k=8"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the files the counted expert-GEMM kernels are compiled from, and their build flags
# (bf16 weights; FP8 weights add their own kernels)
GEMM_SOURCES = ["sparse_moe_layer_affinity_amd/csrc/gemm.hip",
                "sparse_moe_layer_affinity_amd/csrc/gemm_common.h",
                "sparse_moe_layer_affinity_amd/csrc/kernels.h",
                "sparse_moe_layer_affinity_amd/csrc/common.h",
                "include/moe.h",
                "sparse_moe_layer_affinity_amd/build.py"]
GEMM_SOURCES_FP8 = ["sparse_moe_layer_affinity_amd/csrc/gemm_fp8.hip",
                    "sparse_moe_layer_affinity_amd/csrc/gemm_fp8p2.hip"]


def source_hash(fp8: bool) -> str:
    """Hash of the expert-GEMM kernels' sources (with the FP8 kernels' for FP8
    weights), to tell whether stored counter figures of those kernels still apply."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES + (GEMM_SOURCES_FP8 if fp8 else []):
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_record(workload: str, fp8: bool):
    """The committed counter runs (rocprofv3 --pmc) of a workload's expert-GEMM kernels,
    or None when those kernels changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(fp8):
        return None
    return rec


def cpu_baseline(cfg, d, n_tokens: int, n_tokens_1t: int = 8):
    """The oracle as it stands (float64 numpy), on the host cores of this machine:
      * routing of all T tokens of the batch (affinities, bias, group limit, top-K,
        gates), tokens/s;
      * the full layer on n_tokens seeded tokens of the batch (their routing, then the
        shared and the K routed SwiGLU experts and the weighted sum), tokens/s; the
        device-to-host copies of each expert's weights and their widening to float64
        are timed apart and excluded;
      * the same layer leg with BLAS limited to one thread on n_tokens_1t tokens.
    ``value`` is the layer rate (the metric's unit)."""
    import numpy as np
    import oracle
    import workloads
    from threadpoolctl import threadpool_info, threadpool_limits

    bias = d["bias"].cpu().numpy()
    w_r = d["w_router"].cpu()
    x_all = d["x"].cpu()

    def get_expert(fetch):
        def get(e):
            t = time.perf_counter()
            if workloads.is_fp8(cfg.w):
                w = tuple(oracle.dequantize_blocks_128(d[n][e], d["s" + n[1:]][e])
                          for n in ("w_gate", "w_up", "w_down"))
            else:
                w = tuple(d[n][e].to("cpu").double().numpy() for n in ("w_gate", "w_up", "w_down"))
            fetch[0] += time.perf_counter() - t
            return w
        return get

    def layer_leg(n):
        rows = workloads.sample_rows(cfg.T, n, seed=1).numpy()
        x = x_all[rows.tolist()]
        fetch = [0.0]
        t0 = time.perf_counter()
        r = oracle.route(x, w_r, bias, cfg.G, cfg.M, cfg.topn, cfg.K)
        oracle.layer_output(x, r.idx, r.gate, get_expert(fetch), cfg.E, cfg.Ns)
        return n / (time.perf_counter() - t0 - fetch[0]), fetch[0]

    t0 = time.perf_counter()
    oracle.route(x_all, w_r, bias, cfg.G, cfg.M, cfg.topn, cfg.K)
    route_rate = cfg.T / (time.perf_counter() - t0)
    layer_rate, fetch_s = layer_leg(n_tokens)
    with threadpool_limits(limits=1):
        layer_rate_1t, _ = layer_leg(n_tokens_1t)
    blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    cores = min(len(os.sched_getaffinity(0)), max(blas, 1))
    return {"value": round(layer_rate, 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "routing_all_tokens_per_s": round(route_rate, 1),
            "layer_tokens_per_s_1_thread": round(layer_rate_1t, 3),
            "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(blas),
            "sample": f"layer: {n_tokens} seeded tokens of the {cfg.T}-token batch (float64 "
                      f"routing, shared + {cfg.K} routed SwiGLU experts, weighted sum; the "
                      f"{fetch_s:.1f} s of weight copies to the host and widening to float64 "
                      f"excluded); routing: all {cfg.T} tokens; 1 thread: {n_tokens_1t} tokens"}


def calibration_leg(stream):
    """Measured ceilings of this device (calibration kernels of libmoe_calib.so, timed
    between HIP events on the bench stream after the layer steps): a plain read stream
    over 4 GiB (16-byte vectors, eight in flight per lane), a plain write stream over the
    same 4 GiB (16-byte vectors) and back-to-back MFMAs
    (eight accumulator chains per wave, four waves per CU, sustained about 20 ms) in
    bf16 (32x32x16) and e4m3 (32x32x64).  Each is run twice; the second run counts."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_moe_layer_affinity_amd", "libmoe_calib.so"))
    lib.moe_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.moe_calib_write.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.moe_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    s = stream.cuda_stream

    def timed(fn):
        ms = None
        for _ in range(2):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            assert fn() == 0
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1])
        return ms

    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    blocks = 2048
    out = torch.empty(blocks * 256 * 4, dtype=torch.int32, device="cuda")
    ms = timed(lambda: lib.moe_calib_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, s))
    read_gbps = nbytes / (ms * 1e-3) / 1e9
    ms = timed(lambda: lib.moe_calib_write(buf.data_ptr(), nbytes, blocks, s))
    write_gbps = nbytes / (ms * 1e-3) / 1e9
    del buf
    res = {"hbm_read_GBps": round(read_gbps, 1), "hbm_write_GBps": round(write_gbps, 1)}
    iters = 20000
    outf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for name, fp8, flop in (("mfma_bf16_TFLOPs", 0, 32768), ("mfma_e4m3_TFLOPs", 1, 131072)):
        ms = timed(lambda: lib.moe_calib_mfma(fp8, iters, outf.data_ptr(), blocks, s))
        res[name] = round(blocks * 4 * iters * 8 * flop / (ms * 1e-3) / 1e12, 1)
    return res


def library_leg(cfg, stream, reps: int = 5):
    """The vendor library on the expert GEMMs' shapes, for comparison only (not on the
    layer's path): batched bf16 GEMMs through torch.bmm (hipBLASLt / rocBLAS) over E
    experts of ceil(T (K + Ns) / E) rows each, with E distinct weight matrices streamed
    from HBM as in the grouped GEMM: GEMM1 [rows, h] x [h, 2 inter] (gate and up
    together, no SwiGLU) and GEMM2 [rows, inter] x [inter, h]; row-major operands,
    both contiguous.  No gather, no SwiGLU, no ragged rows: an easier problem than the
    grouped FFN's.  Timed between HIP events, ``reps`` calls after one warm-up."""
    import torch
    E, H, I = cfg.E, cfg.hidden, cfg.inter
    m = -(-cfg.T * (cfg.K + cfg.Ns) // E)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    res = {"batch": E, "rows_per_expert": m}
    for name, k, n in (("gemm1", H, 2 * I), ("gemm2", I, H)):
        a = (torch.randn((E, m, k), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        b = (torch.randn((E, k, n), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        out = torch.empty((E, m, n), dtype=torch.bfloat16, device="cuda")
        torch.bmm(a, b, out=out)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            torch.bmm(a, b, out=out)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        flops = 2.0 * E * m * k * n
        res[name + "_ms"] = round(ms, 4)
        res[name + "_TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 1)
        del a, b, out
    return res


def balance_loss_leg(moe, cfg, c, d, idx, ws, stream, reps: int = 20):
    """Time the training-side extras outside the layer step: moe_router_scores and
    moe_balance_loss (two sequences of T/2 tokens, with f, P and the logit gradient),
    each over ``reps`` back-to-back calls between HIP events on the bench stream.
    The loss's algorithmic bytes: affinities and selections read once, the gradient
    written once, plus the per-sequence f, P and loss."""
    import torch
    T, E, K = cfg.T, cfg.E, cfg.K
    L = T // 2
    S = T // L
    scores = torch.empty((T, E), dtype=torch.float32, device="cuda")
    loss = torch.empty(S, dtype=torch.float32, device="cuda")
    frac = torch.empty((S, E), dtype=torch.float32, device="cuda")
    prob = torch.empty((S, E), dtype=torch.float32, device="cuda")
    grad = torch.empty((T, E), dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / reps

    us_scores = timed(lambda: moe.moe_router_scores(c, d["x"], d["w_router"], scores, ws))
    us_loss = timed(lambda: moe.moe_balance_loss(c, scores, idx, L, 1e-4, loss, frac, prob, grad,
                                                 ws))
    nbytes = T * E * 4 + T * K * 4 + T * E * 4 + S * E * 8 + S * 4
    gbps = nbytes / (us_loss * 1e-6) / 1e9
    return {"seq_len": L, "alpha": 1e-4, "router_scores_us": round(us_scores, 2),
            "loss_and_grad_us": round(us_loss, 2), "loss_bytes": nbytes,
            "loss_GBps": round(gbps, 1), "loss_frac_hbm": round(gbps / HBM_PEAK, 4),
            "loss_value": [round(float(v), 9) for v in loss.cpu()]}


def backward_leg(moe, cfg, c, d, idx, gate, offsets, row_token, pair_row, y_rows, y, ws, stream,
                 reps: int = 20):
    """Time the combine, gate and SwiGLU backward outside the layer step: the first two
    on the step's own y_rows, routing and permutation, with the layer output standing
    in for the output gradient.  Algorithmic bytes: combine backward reads dy and the
    routed rows once and writes every row gradient once (plus dgate, pair_row and the
    gates); gate backward reads K affinities, indices and gate gradients per token and
    writes the [T, E] logit gradient; SwiGLU backward reads three [rows, inter] arrays
    and writes two.  The experts' input gradient (bf16) is timed on the step's own
    inputs and the combine backward's row gradients, reported with its GEMM FLOPs, and
    their weight gradients with the a, b and dh GEMMs they need, both in one call (a, b
    and dh shared: 14 rows H I flops), and the router logits' backward (dx and dW_r,
    4 T E H flops)."""
    import torch
    T, E, K, H = cfg.T, cfg.E, cfg.K, cfg.hidden
    eb = 4 if cfg.act == "f32" else 2
    dgate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dy_rows = torch.empty_like(y_rows)
    scores = torch.empty((T, E), dtype=torch.float32, device="cuda")
    grad = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_router_scores(c, d["x"], d["w_router"], scores, ws)

    def timed(fn, n=reps):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(n):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / n

    us_comb = timed(lambda: moe.moe_combine_backward(c, y, y_rows, pair_row, gate, dgate, dy_rows))
    us_gate = timed(lambda: moe.moe_gate_backward(c, scores, idx, dgate, grad))
    us_rb = None
    if cfg.act != "f32":
        dxr = torch.empty((T, H), device="cuda")
        dwr = torch.empty((E, H), device="cuda")
        rws = torch.empty(moe.moe_router_backward_workspace_bytes(c), dtype=torch.uint8,
                          device="cuda")
        us_rb = timed(lambda: moe.moe_router_backward(c, d["x"], d["w_router"], grad, dxr, dwr,
                                                      rws))
        del dxr, dwr, rws
    # SwiGLU backward over every grouped row: seeded stand-ins for the pre-activations
    # and the gradient of h (the forward does not keep the pre-activations)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    shape = (cfg.rows, cfg.inter)
    adt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    pre_a = (2.0 * torch.randn(shape, generator=g, device="cuda")).to(adt)
    pre_b = torch.randn(shape, generator=g, device="cuda").to(adt)
    dh = torch.randn(shape, generator=g, device="cuda").to(adt)
    da, db = torch.empty_like(pre_a), torch.empty_like(pre_a)
    us_swi = timed(lambda: moe.moe_swiglu_backward(c, pre_a, pre_b, dh, cfg.rows, da, db))
    b_swi = 5 * cfg.rows * cfg.inter * eb
    gb_swi = b_swi / (us_swi * 1e-6) / 1e9
    del pre_a, pre_b, dh, da, db
    # input gradient of the experts (bf16 only): the step's own x, permutation and
    # weights, the combine backward's row gradients
    ex = None
    need = moe.moe_backward_workspace_bytes(c)
    if need:
        bws = torch.empty(need, dtype=torch.uint8, device="cuda")
        dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        wts = {k: d[k] for k in ("w_gate", "w_up", "w_down")}
        us_ex = timed(lambda: moe.moe_expert_backward_input(c, d["x"], offsets, row_token, pair_row,
                                                            wts, dy_rows, dx, bws), n=5)
        G = cfg.E + cfg.Ns
        dwg = torch.empty((G, cfg.inter, H), device="cuda")
        dwu = torch.empty_like(dwg)
        dwd = torch.empty((G, H, cfg.inter), device="cuda")
        us_w = timed(lambda: moe.moe_expert_backward(c, d["x"], offsets, row_token, pair_row, wts,
                                                     dy_rows, None, dwg, dwu, dwd, bws), n=2)
        # both gradients in one call (a, b and dh computed once for both)
        us_full = timed(lambda: moe.moe_expert_backward(c, d["x"], offsets, row_token, pair_row,
                                                        wts, dy_rows, dx, dwg, dwu, dwd, bws), n=2)
        del dwg, dwu, dwd
        flops_w = 6.0 * cfg.rows * H * cfg.inter      # three weight gradients: 2 r H I each
        flops = 8.0 * cfg.rows * H * cfg.inter        # a, b, dh: 2 r H I each; dX: 4 r H I
        ex = {"expert_backward_input_us": round(us_ex, 1),
              "expert_backward_input_gemm_flops": flops,
              "expert_backward_input_tflops": round(flops / (us_ex * 1e-6) / 1e12, 1),
              "expert_backward_weights_us": round(us_w, 1),
              "expert_backward_weights_flops": flops_w + 6.0 * cfg.rows * H * cfg.inter,
              "expert_backward_weights_tflops": round(
                  (flops_w + 6.0 * cfg.rows * H * cfg.inter) / (us_w * 1e-6) / 1e12, 1),
              "expert_backward_full_us": round(us_full, 1),
              "expert_backward_full_flops": flops + flops_w,
              "expert_backward_full_tflops": round((flops + flops_w) / (us_full * 1e-6) / 1e12, 1)}
        del bws
    b_comb = T * H * eb + T * K * H * eb + cfg.rows * H * eb + T * K * (4 + 8)
    b_gate = T * K * 12 + T * E * 4
    gb_comb = b_comb / (us_comb * 1e-6) / 1e9
    gb_gate = b_gate / (us_gate * 1e-6) / 1e9
    return {"combine_backward_us": round(us_comb, 2), "combine_backward_bytes": b_comb,
            "combine_backward_GBps": round(gb_comb, 1),
            "combine_backward_frac_hbm": round(gb_comb / HBM_PEAK, 4),
            "gate_backward_us": round(us_gate, 2), "gate_backward_bytes": b_gate,
            "gate_backward_GBps": round(gb_gate, 1),
            "router_backward_us": None if us_rb is None else round(us_rb, 1),
            "router_backward_tflops": None if us_rb is None else
            round(4.0 * T * E * H / (us_rb * 1e-6) / 1e12, 1),
            "swiglu_backward_us": round(us_swi, 2), "swiglu_backward_bytes": b_swi,
            "swiglu_backward_GBps": round(gb_swi, 1),
            "swiglu_backward_frac_hbm": round(gb_swi / HBM_PEAK, 4), **(ex or {})}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_bf16",
                    choices=["prefill_bf16", "decode_bf16", "prefill_fp8", "prefill_fp8_pow2", "skewed_bf16"])
    ap.add_argument("--cpu-tokens", type=int, default=48,
                    help="tokens in the oracle's bounded sample (0 skips it)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the layer steps only (no calibration kernels, balance loss or "
                         "backward legs after them), e.g. for counter runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")      # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; the layer's sharding is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_moe_layer_affinity_amd as moe
    import workloads

    cfg = workloads.get(args.workload)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    log(f"[bench] generating {cfg.name} inputs on the GPU")
    d = workloads.make_layer_inputs(cfg, device="cuda")
    c = moe.make_config(cfg.T, cfg.hidden, cfg.inter, cfg.E, cfg.K, cfg.G, cfg.M, cfg.topn,
                        cfg.Ns, cfg.act, cfg.w)
    ws = torch.empty(moe.moe_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    adt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    T, K, E = cfg.T, cfg.K, cfg.E
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    load = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_token = torch.empty(T * K, dtype=torch.int32, device="cuda")
    pair_row = torch.empty(T * K, dtype=torch.int32, device="cuda")
    y_rows = torch.empty((cfg.rows, cfg.hidden), dtype=adt, device="cuda")
    y = torch.empty((T, cfg.hidden), dtype=adt, device="cuda")
    bias = d["bias"].clone()
    weights = {k: d[k] for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down") if k in d}
    stages = ["route", "permute", "grouped_ffn", "combine", "bias_update"]
    n_all = args.warmup + args.steps
    # every step writes its loads to a buffer of its own (read after the timed region);
    # the skewed workload draws a fresh seeded batch per step (the balancing loop of its
    # configuration), generated before the timed region and resident in HBM
    loads = torch.empty((n_all, E), dtype=torch.int32, device="cuda")
    fresh = cfg.steps > 1
    batches = [d["x"]] + ([workloads.make_tokens(cfg, step=s, device="cuda")
                           for s in range(1, n_all)] if fresh else [])

    def step(i, ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record(stream)
        x = batches[i] if fresh else d["x"]
        load = loads[i]
        mark(0)
        moe.moe_route(c, x, d["w_router"], bias, idx, gate, ws)
        mark(1)
        moe.moe_permute(c, idx, load, offsets, row_token, pair_row, ws)
        mark(2)
        moe.moe_grouped_ffn(c, x, offsets, row_token, weights, y_rows, ws)
        mark(3)
        moe.moe_combine(c, y_rows, pair_row, gate, None, y)
        mark(4)
        moe.moe_bias_update(c, load, cfg.gamma, bias)
        mark(5)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed_loads = loads[args.warmup:].cpu().numpy()
    load = loads[n_all - 1]
    d["x"] = batches[n_all - 1] if fresh else d["x"]       # the last step's batch, for the extras

    stage_ms = {st: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                                   for s in range(args.steps)])) for i, st in enumerate(stages)}
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T / (elapsed / args.steps)

    ffn_flops = 6.0 * cfg.hidden * cfg.inter * T * (K + cfg.Ns)      # real rows only
    ffn_ms = stage_ms["grouped_ffn"]
    gemm_tflops = ffn_flops / (ffn_ms * 1e-3) / 1e12
    # algorithmic bytes of each timed step: the weights of the experts that step touched
    # (the bias moves every step, so the set does) + x read + the rows written once
    touched = (timed_loads > 0).sum(1) + cfg.Ns                          # [steps]
    wbytes_per_elem = 1 if workloads.is_fp8(cfg.w) else (4 if cfg.w == "f32" else 2)
    per_expert = 3 * cfg.hidden * cfg.inter * wbytes_per_elem
    if workloads.is_fp8(cfg.w):
        per_expert += 3 * (cfg.hidden // 128) * (cfg.inter // 128) * 4
    ab = 4 if cfg.act == "f32" else 2
    ffn_bytes = float(np.mean(touched)) * per_expert + 2 * T * cfg.hidden * ab
    # the layer's: + the router weight, the bias, indices, gates and loads
    layer_bytes = ffn_bytes + E * cfg.hidden * ab + E * 8 + T * K * 8
    decode = cfg.T <= 512
    # the bound: whichever of the FLOPs at the dense MFMA peak and the algorithmic bytes
    # at the HBM peak takes longer (the prefill GEMMs sit just on the HBM side of the
    # ridge: about 280 FLOP per byte against 2500 / 8 = 312)
    gb_s = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    t_mfma = ffn_flops / (PEAK[cfg.w] * 1e12)
    t_hbm = ffn_bytes / (HBM_PEAK * 1e9)
    hbm_bound = decode or t_hbm > t_mfma
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gb_s, 1), "peak": HBM_PEAK, "unit": "GB/s",
                "frac": round(gb_s / HBM_PEAK, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK[cfg.w],
                "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK[cfg.w], 4)}
    roof["mfma_frac"] = round(gemm_tflops / PEAK[cfg.w], 4)
    roof["hbm_frac"] = round(gb_s / HBM_PEAK, 4)
    roof["ms_at_mfma_peak"] = round(t_mfma * 1e3, 4)
    roof["ms_at_hbm_peak"] = round(t_hbm * 1e3, 4)
    if decode:
        lay = layer_bytes / (ms_per_step * 1e-3) / 1e9
        roof["layer"] = {"achieved": round(lay, 1), "frac": round(lay / HBM_PEAK, 4),
                         "bytes": layer_bytes, "ms": round(ms_per_step, 4)}
    stored = stored_record(cfg.name, workloads.is_fp8(cfg.w))
    roof["traffic"] = stored["bytes_per_launch"] if stored else None
    roof["kernel"] = "moe_grouped_ffn (grouped_gemm gated GEMM1 + GEMM2)"
    roof["algorithmic"] = {"flops": ffn_flops, "bytes": ffn_bytes,
                           "touched_experts_per_step": [int(v) for v in touched]}
    if stored:
        roof["counters"] = stored["kernels"]

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3" if workloads.is_fp8(cfg.w) else "bf16",
        "data": "synthetic (seeded; weights N(0, 0.02^2), x N(0, 1))",
        "config": {"workload": cfg.name, "T": T, "hidden": cfg.hidden, "inter": cfg.inter,
                   "E": E, "K": K, "G": cfg.G, "M": cfg.M, "group_topn": cfg.topn,
                   "shared": cfg.Ns, "act": cfg.act, "weights": cfg.w},
        "grouped_gemm_tflops": round(gemm_tflops, 1),
        "grouped_gemm_frac_of_peak": round(gemm_tflops / PEAK[cfg.w], 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "max_over_mean_load": round(float(load.max().item()) / (T * K / E), 3),
        "roofline": roof,
    }
    if fresh:
        # the balancing loop: max/mean load of every step, warm-up steps first
        mean_load = T * K / E
        result["balancing"] = {
            "steps": n_all, "gamma": cfg.gamma, "fresh_batch_per_step": True,
            "max_over_mean_load_per_step": [round(float(v) / mean_load, 3)
                                            for v in loads.max(1).values.cpu().numpy()]}

    if not args.no_extras:
        cal = calibration_leg(stream)
        if cfg.act == "bf16" and cfg.w == "bf16":
            cal["library_bmm_bf16"] = library_leg(cfg, stream)
        result["calibration"] = cal
        measured = cal["hbm_read_GBps"] if hbm_bound else cal[
            "mfma_e4m3_TFLOPs" if workloads.is_fp8(cfg.w) else "mfma_bf16_TFLOPs"]
        roof["measured_peak"] = measured
        roof["frac_of_measured_peak"] = round(roof["achieved"] / measured, 4)
        result["balance_loss"] = balance_loss_leg(moe, cfg, c, d, idx, ws, stream)
        result["backward"] = backward_leg(moe, cfg, c, d, idx, gate, offsets, row_token, pair_row,
                                          y_rows, y, ws, stream)
        result["backward"]["expert_wgrad_fp32_out_bytes"] = 4.0 * 3 * (E + cfg.Ns) * cfg.hidden * cfg.inter
    if args.cpu_tokens > 0:
        log(f"[bench] oracle baseline on {args.cpu_tokens} tokens")
        result["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_tokens)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
