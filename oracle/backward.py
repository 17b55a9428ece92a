"""Plain float64 oracle of the combine and gate backward (test infrastructure only).

Source (the pages): "DeepSeek-V3 Technical Report 深度解读报告", section 2.2: the
layer output is the token's input plus the shared experts' outputs plus the routed
experts' outputs weighted by gates g_k = s_k / sum_j s_j (s the sigmoid affinities
of the selected experts); section 2.3: the bias b only decides the selection and
does not enter the gates.  The backward is the adjoint of these formulas (the pages
state no backward; differentiating them is the plain reading):

  combine      y_t = [u_t] + sum_s Y[shared row of t] + sum_k g_tk Y[pair_row(t, k)]
  adjoint      dg_tk = <dy_t, Y[pair_row(t, k)]>
               dY[pair_row(t, k)] = g_tk dy_t ;  dY[shared row of t] = dy_t
  gates        g_k = s_k / S,  S = sum_j s_{idx_j}
               dL/ds_j = (dg_j - sum_k dg_k g_k) / S     for the selected j, 0 elsewhere
               dL/dz_j = dL/ds_j * s_j (1 - s_j)          (s = sigmoid(z))
  bias         no gradient: the selection is piecewise constant in b.

SwiGLU expert ("深度解读报告" section 2.2 with SwiGLU experts, the reading of the
garbled activation passage): h = silu(a) * b with a = W_gate u, b = W_up u and
silu(a) = a sigmoid(a); its backward for an upstream gradient dh is
  da = dh * b * silu'(a),  silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a)))
  db = dh * silu(a).

Parity status: pinned by mathematics.  The combine adjoint by the adjoint identity
<dy, C(Y, g)> = <dY, Y> + <dg, g> (C is linear in Y for fixed g and in g for fixed Y)
and by a hand-computed case; the gate backward by central finite differences of the
gates, a hand-computed case, and a closed form (a dg equal over k gives no gradient,
because the gates sum to one); the SwiGLU backward by central finite differences of
sum(dh * h) and the closed forms at a = 0 (silu' = 1/2, silu = 0); the expert input
gradient by central finite differences of sum_r <dy_r, FFN_e(x_t)> with respect to x
and by linearity in dy; the expert weight gradients by central finite differences of
the same sum with respect to weight entries; the router backward by the adjoint
identity <dz, x' W_r^T> = <dx, x'> and <dz, x W'^T> = <dW_r, W'>.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def combine_backward(dy, y_rows, pair_row, gate, num_tokens: int, top_k: int,
                     num_shared: int):
    """Adjoint of the combine.  dy [T, h]; y_rows [T*K + T*Ns, h] (routed rows, then
    each shared expert's T rows in token order); pair_row [T*K]; gate [T, K].
    Returns (dgate [T, K], dy_rows [T*K + T*Ns, h]) in float64."""
    dy = _f64(dy)
    Y = _f64(y_rows)
    g = _f64(gate)
    pair_row = np.asarray(pair_row, dtype=np.int64)
    T, K, Ns = num_tokens, top_k, num_shared
    TK = T * K
    dgate = np.zeros((T, K))
    dY = np.zeros_like(Y)
    for t in range(T):
        for k in range(K):
            r = pair_row[t * K + k]
            dgate[t, k] = np.dot(dy[t], Y[r])
            dY[r] = g[t, k] * dy[t]
        for s in range(Ns):
            dY[TK + s * T + t] = dy[t]
    return dgate, dY


def gate_backward(z, idx, dgate) -> np.ndarray:
    """Gradient with respect to the router logits z [T, E] of a loss whose gradient
    with respect to the gates is dgate [T, K], the selection idx [T, K] held fixed."""
    z = _f64(z)
    s = 1.0 / (1.0 + np.exp(-z))
    idx = np.asarray(idx, dtype=np.int64)
    dg = _f64(dgate)
    T, _ = z.shape
    grad = np.zeros_like(z)
    for t in range(T):
        sel = s[t, idx[t]]
        total = sel.sum()
        g = sel / total
        ds = (dg[t] - np.dot(dg[t], g)) / total
        grad[t, idx[t]] = ds * sel * (1.0 - sel)
    return grad


def swiglu_backward(a, b, dh):
    """Gradients (da, db) of sum(dh * silu(a) * b) with respect to the gate and up
    pre-activations a and b (any equal shapes), float64."""
    a = _f64(a)
    b = _f64(b)
    dh = _f64(dh)
    sig = 1.0 / (1.0 + np.exp(-a))
    silu = a * sig
    dsilu = sig * (1.0 + a * (1.0 - sig))
    return dh * b * dsilu, dh * silu


def expert_input_backward(x, row_token, num_tokens: int, top_k: int, num_shared: int,
                          dy_rows, get_expert, expert_of_row):
    """Input gradient of the grouped SwiGLU experts: for every grouped row r of expert
    e = expert_of_row[r] (token t = row_token[r] for routed rows, r - T*K mod T for
    the shared rows), with u = x[t], a = W_gate u, b = W_up u, h = silu(a) * b and
    y_r = W_down h,
      dh = W_down^T dy_rows[r],  (da, db) = swiglu_backward(a, b, dh),
      dX[r] = W_gate^T da + W_up^T db,   dx[t] = sum of dX over the token's rows.
    get_expert(e) -> (w_gate [I, H], w_up [I, H], w_down [H, I]).  Returns
    (dX [rows, H], dx [T, H]) in float64; rows of experts never named are skipped."""
    x = _f64(x)
    dY = _f64(dy_rows)
    T, K, Ns = num_tokens, top_k, num_shared
    TK = T * K
    rows = dY.shape[0]
    tok = np.array([row_token[r] if r < TK else (r - TK) % T for r in range(rows)])
    expert_of_row = np.asarray(expert_of_row)
    dX = np.zeros((rows, x.shape[1]))
    for e in np.unique(expert_of_row):
        rs = np.nonzero(expert_of_row == e)[0]
        wg, wu, wd = (_f64(m) for m in get_expert(int(e)))
        u = x[tok[rs]]
        a = u @ wg.T
        b = u @ wu.T
        dh = dY[rs] @ wd
        da, db = swiglu_backward(a, b, dh)
        dX[rs] = da @ wg + db @ wu
    dx = np.zeros((T, x.shape[1]))
    for r in range(rows):
        dx[tok[r]] += dX[r]
    return dX, dx


def expert_weight_backward(x, row_token, num_tokens: int, top_k: int, dy_rows, get_expert,
                           expert_of_row, experts):
    """Weight gradients of the grouped SwiGLU experts: for each expert e in `experts`,
    over its rows r (u = x[token of r], a = W_gate u, b = W_up u, h = silu(a) b),
      dW_down[e] = sum_r dy_r h_r^T,   dW_gate[e] = sum_r da_r u_r^T,
      dW_up[e]   = sum_r db_r u_r^T,   (da, db) = swiglu_backward(a, b, W_down^T dy_r).
    Returns {e: (dW_gate [I, H], dW_up [I, H], dW_down [H, I])} in float64."""
    x = _f64(x)
    dY = _f64(dy_rows)
    T, K = num_tokens, top_k
    TK = T * K
    expert_of_row = np.asarray(expert_of_row)
    out = {}
    for e in experts:
        rs = np.nonzero(expert_of_row == e)[0]
        wg, wu, wd = (_f64(m) for m in get_expert(int(e)))
        tok = np.array([row_token[r] if r < TK else (r - TK) % T for r in rs], dtype=np.int64)
        u = x[tok] if len(rs) else np.zeros((0, x.shape[1]))
        a = u @ wg.T
        b = u @ wu.T
        h = a / (1.0 + np.exp(-a)) * b
        dh = dY[rs] @ wd
        da, db = swiglu_backward(a, b, dh)
        out[int(e)] = (da.T @ u, db.T @ u, dY[rs].T @ h)
    return out


def router_backward(x, w_router, grad_logits):
    """Backward of the router logits z = x W_r^T for a logit gradient dz [T, E]:
    dx = dz W_r [T, H] and dW_r = dz^T x [E, H], float64."""
    x = _f64(x)
    w = _f64(w_router)
    dz = _f64(grad_logits)
    return dz @ w, dz.T @ x

