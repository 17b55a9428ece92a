"""CPU oracle for the DeepSeekMoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports, links or calls it, and this package imports
nothing from the product.  The two share no code; only the seeded input
generators in ``workloads`` feed both.

Everything here is a plain, slow, float64 restatement of what the pages say the
layer computes (sources: "DeepSeek-V3 Technical Report 深度解读报告", sections
2.2 DeepSeekMoE, 2.3 Auxiliary-Loss-Free Load Balancing, 2.4 Node-Limited
Routing; "DeepSeek-V3 ... 技术解析" (devpress), section 1 on 256 routed + 1 shared
experts with top-8, section 2 on 128x128 / 1x128 FP8 block quantisation; the
e4m3 maximum of 448 from the stapisi blog, section 6.2).  Where a step decides an
integer from floating point (top-K selection, an FP8 code), the decision is
taken in float32, the precision of the kernels; everything else is float64.

Parity status per function (what pins it; the tests under ``tests/`` hold the pins):
  route            pinned: brute-force subset enumeration, torch.topk special case
                   (M = G), invariants (K distinct experts, <= M groups, gates sum
                   to 1, constant bias shift is a no-op, b = 0 gives top-K of z)
  permute          pinned: pure-Python counting/placement on tiny inputs, invariants
  expert_ffn       pinned: pure-Python triple loop on tiny shapes, zero-W_up case
  layer_output     pinned: one-hot gate reduces to one expert, dense-mixture case,
                   linearity in the shared expert
  bias_update      pinned: closed form of the +-gamma rule, hand-written golden file
  e4m3 table/RNE   pinned: all 256 codes and a float32 sweep vs torch.float8_e4m3fn
  quantize_1x128   pinned: bound |x - s*q| <= half an e4m3 step, amax maps to 448,
                   zero block gets scale 1, hand-computed golden rows
  pow2_scale /     pinned: power of two, amax <= 448 s < 2 amax (brute force over a
  quantize_1x128_pow2      float32 sweep against an integer-exponent search), hand
                   values (448 -> 1, 449 -> 2, 1 -> 2^-8), blocks of e4m3 values times
                   a power of two quantise exactly, the half-step bound
  expert_ffn_fp8_  pinned: a hand-worked one-token expert over two 1x128 tiles in each
  emulated (and    GEMM, every e4m3 code and scale derived by hand (both scale rules);
  _pow2_emulated)  planted mistakes (h or x left unquantised, no bf16 rounding of h,
                   power-of-two scales on the amax/448 path, one scale per row, gate
                   and up swapped) each move a hand-derived output
  balance_loss /   formula is a reading (the pages name the sequence-wise loss but
  balance_loss_    print no formula): pinned by hand-computed cases, the closed
  grad_logits      forms of perfect balance, uniform affinities and full
                   concentration, sum f = E and sum P = 1, relabelling and
                   per-sequence locality, and central finite differences
  combine_backward pinned: the adjoint identity of the combine (linear in the rows
                   and in the gates), a hand-computed case
  gate_backward    pinned: central finite differences of the gates, a hand-computed
                   case, zero gradient for a dgate equal over the selection and for
                   unselected experts
  swiglu_backward  pinned: central finite differences, the closed forms at a = 0
  expert_input_    pinned: central finite differences of sum_r <dy_r, FFN(x_t)> in x,
  backward         linearity in dy
  expert_weight_   pinned: central finite differences of the same sum in the weights
  backward
  router_backward  pinned: the adjoint identities of z = x W_r^T in x and in W_r
"""
from .moe_layer import (RouteResult, affinities, route, select, valid_selections, permute, expert_ffn, layer_output,
                        bias_update, silu)
from .backward import (combine_backward, expert_input_backward, expert_weight_backward,
                       gate_backward, router_backward, swiglu_backward)
from .balance import balance_loss, balance_loss_grad_logits
from .e4m3 import (e4m3_table, e4m3_encode_rne, quantize_1x128, dequantize_1x128,
                   dequantize_blocks_128, expert_ffn_fp8_emulated, pow2_scale,
                   quantize_1x128_pow2, expert_ffn_fp8_pow2_emulated)

__all__ = ["RouteResult", "affinities", "route", "select", "valid_selections", "permute", "expert_ffn", "layer_output",
           "bias_update", "silu", "e4m3_table", "e4m3_encode_rne", "quantize_1x128",
           "dequantize_1x128", "dequantize_blocks_128", "expert_ffn_fp8_emulated", "pow2_scale", "quantize_1x128_pow2", "expert_ffn_fp8_pow2_emulated",
           "balance_loss", "balance_loss_grad_logits", "combine_backward", "gate_backward",
           "swiglu_backward", "expert_input_backward", "expert_weight_backward",
           "router_backward"]
