"""Plain float64 oracle of the sequence-wise balance loss (test infrastructure only).

Source (the pages): "DeepSeek-V3 Technical Report 深度解读报告", section 2.3
(Auxiliary-Loss-Free Load Balancing): beside the bias rule, a sequence-level
balance loss L_Bal with a very small coefficient alpha guards against extreme
imbalance inside a single sequence; section 4.4 compares a sequence-wise with a
batch-wise auxiliary loss.  The pages name the loss but print no formula.

Reading (the plainest form consistent with those passages, and the one the
DeepSeek-V3 technical report itself defines), per sequence of T_s tokens, over the
N_r routed experts, with K_r experts selected per token:

  s'_{i,t} = s_{i,t} / sum_j s_{j,t}                 affinities normalised per token
  f_i      = N_r / (K_r T_s) * #{t : expert i selected for token t}
  P_i      = (1 / T_s) * sum_t s'_{i,t}
  L        = alpha * sum_i f_i P_i

"Selected" is the routing decision of the layer (the top-K indices, group limit and
selection bias included).  The batch-wise variant is the same loss with the whole
batch as one sequence (T_s = T).  f is piecewise constant in the affinities, so the
gradient reaches the logits z only through P:

  dL/ds'_{i,t} = alpha f_i / T_s
  dL/ds_{j,t}  = (alpha / T_s) (f_j - sum_i f_i s'_{i,t}) / sum_k s_{k,t}
  dL/dz_{j,t}  = dL/ds_{j,t} * s_{j,t} (1 - s_{j,t})        (s = sigmoid(z))

Parity status: the formula is a reading (the pages print none), so the loss is
pinned by mathematics, not by a worked example of the pages: a hand-computed case,
the closed forms of perfect balance (L = alpha) and full concentration
(L = alpha N_r / K_r), uniform affinities (L = alpha for any selection), the
invariants sum_i f_i = N_r and sum_i P_i = 1, invariance under relabelling the
experts, locality per sequence, and central finite differences of the loss for the
gradient.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def balance_loss(s, idx, seq_len: int, alpha: float, top_k: int):
    """Per-sequence balance loss from affinities s [T, E] and selections idx [T, K].

    Tokens [q*seq_len, (q+1)*seq_len) form sequence q; seq_len must divide T.
    Returns (loss [S], f [S, E], P [S, E]) in float64.
    """
    s = _f64(s)
    idx = np.asarray(idx, dtype=np.int64)
    T, E = s.shape
    assert idx.shape == (T, top_k) and T % seq_len == 0
    S = T // seq_len
    s_norm = s / s.sum(axis=1, keepdims=True)
    loss = np.zeros(S)
    f = np.zeros((S, E))
    P = np.zeros((S, E))
    for q in range(S):
        rows = slice(q * seq_len, (q + 1) * seq_len)
        count = np.bincount(idx[rows].ravel(), minlength=E)
        f[q] = E / (top_k * seq_len) * count
        P[q] = s_norm[rows].sum(axis=0) / seq_len
        loss[q] = alpha * np.dot(f[q], P[q])
    return loss, f, P


def balance_loss_grad_logits(z, idx, seq_len: int, alpha: float, top_k: int) -> np.ndarray:
    """Gradient of sum_q L_q with respect to the router logits z [T, E], the
    selection idx held fixed (it is piecewise constant in z)."""
    z = _f64(z)
    s = 1.0 / (1.0 + np.exp(-z))
    _, f, _ = balance_loss(s, idx, seq_len, alpha, top_k)
    T, _ = s.shape
    grad = np.zeros_like(s)
    for t in range(T):
        q = t // seq_len
        total = s[t].sum()
        weighted = np.dot(f[q], s[t] / total)
        ds = (alpha / seq_len) * (f[q] - weighted) / total
        grad[t] = ds * s[t] * (1.0 - s[t])
    return grad
