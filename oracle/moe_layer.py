"""Plain float64 oracle of the DeepSeekMoE layer forward (test infrastructure only).

Sources (the pages):
  [R] "DeepSeek-V3 Technical Report 深度解读报告", section 2.2 (layer formula and
      sigmoid gating normalised over the selected experts), section 2.3 (per-expert
      bias used only for top-K selection, +-gamma update from the whole batch's
      loads at the end of each step), section 2.4 (each token reaches at most M
      nodes, chosen by the sum of the highest affinities on each node; no token
      dropping).
  [D] "DeepSeek-V3 ... 技术解析" (devpress), section 1: 256 routed experts + 1
      shared expert, 8 routed experts per token.

Readings where the pages are silent (each listed in the design notes):
  * affinity logit z_e = <x_t, W_r[e]> (a dot product with expert e's router row)
  * groups are contiguous blocks of E/G experts; a group's score is the sum of its
    ``topn`` largest *biased* affinities
  * two stages: keep the M best groups, then the K best experts among them
  * ties go to the lower group / expert index; the selected list is ordered by
    (biased affinity descending, index ascending)
  * selection decisions are taken on float32-rounded affinities (the kernels'
    precision); near-ties whose float64 gap is below 1e-6 are flagged
  * expert FFN is SwiGLU: W_down (silu(W_gate u) * (W_up u)), silu(a) = a sigmoid(a)
  * shared experts enter with weight 1, routed experts with their gate, no scaling
  * "overloaded" means load * E > T * K (above the mean), "underloaded" below it
"""
from __future__ import annotations

import dataclasses

import numpy as np

NEAR_TIE = 1e-6


def _f64(a) -> np.ndarray:
    """Exact widening of a float array (numpy or torch, any float dtype) to float64."""
    if hasattr(a, "detach"):           # torch tensor: bf16 / fp8 have no numpy dtype
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a))."""
    return a / (1.0 + np.exp(-a))


def affinities(x, w_router) -> tuple[np.ndarray, np.ndarray]:
    """Token-to-expert logits and sigmoid affinities ([R] section 2.2).

    x [T, h], w_router [E, h] -> z [T, E] = x W_r^T and s = 1 / (1 + exp(-z)), float64.
    """
    z = _f64(x) @ _f64(w_router).T
    return z, 1.0 / (1.0 + np.exp(-z))


@dataclasses.dataclass
class RouteResult:
    idx: np.ndarray            # [T, K] int32 selected experts, (sb desc, index asc)
    gate: np.ndarray           # [T, K] float64 gates s / sum(s) over the selection
    s: np.ndarray              # [T, E] float64 affinities
    sb: np.ndarray             # [T, E] float64 biased affinities (selection only)
    groups: np.ndarray         # [T, M] int32 kept groups, (score desc, index asc)
    near_tie_group: np.ndarray     # [T] bool: M-th / (M+1)-th group score gap < 1e-6
    near_tie_expert: np.ndarray    # [T] bool: K-th / (K+1)-th candidate gap < 1e-6
    near_tie_order: np.ndarray     # [T] bool: two selected experts within 1e-6

    @property
    def near_tie(self) -> np.ndarray:
        """Tokens whose selected *set* may legitimately differ from the kernel's."""
        return self.near_tie_group | self.near_tie_expert


def _top_sum_f32(v32: np.ndarray, n: int) -> np.ndarray:
    """Sum of the n largest float32 values along the last axis, added largest first
    in float32 arithmetic."""
    desc = -np.sort(-v32, axis=-1)
    acc = np.zeros(v32.shape[:-1], np.float32)
    for i in range(n):
        acc = (acc + desc[..., i]).astype(np.float32)
    return acc


def _gap_at(values: np.ndarray, order: np.ndarray, pos: int) -> np.ndarray:
    """values[order[pos-1]] - values[order[pos]] per row (float64)."""
    a = np.take_along_axis(values, order[:, pos - 1:pos], 1)[:, 0]
    b = np.take_along_axis(values, order[:, pos:pos + 1], 1)[:, 0]
    return np.abs(a - b)


def route(x, w_router, bias, num_groups: int, top_groups: int, group_topn: int,
          top_k: int) -> RouteResult:
    """Group-limited top-K routing with a selection-only bias ([R] 2.2, 2.3, 2.4).

    Per token t:
      s_e  = sigmoid(z_te)                         (affinity)
      sb_e = s_e + b_e                             (bias, selection only)
      group j covers experts [j E/G, (j+1) E/G); score_j = sum of its group_topn largest sb
      keep the top_groups groups with the largest score
      select the top_k experts by sb among the kept groups' experts
      gate_k = s_{idx_k} / sum_j s_{idx_j}         (unbiased affinities)
    Selection decisions use float32 s and sb (float32 add of the float32 bias) and a
    float32 group-score sum; gates and near-tie gaps use float64.  Orderings are
    stable sorts of the negated keys, so equal keys keep the lower index first.
    All tokens are processed at once; rows are independent.
    """
    return select(affinities(x, w_router)[1], bias, num_groups, top_groups, group_topn, top_k)


def select(s: np.ndarray, bias, num_groups: int, top_groups: int, group_topn: int,
           top_k: int) -> RouteResult:
    """The selection steps of ``route`` on given float64 affinities s [T, E] (so that
    several biases can be tried on one batch without recomputing the logits)."""
    T, E = s.shape
    G, M, K = num_groups, top_groups, top_k
    n = E // G
    b32 = np.asarray(bias, dtype=np.float32).reshape(E)
    sb = s + b32.astype(np.float64)
    sb32 = (s.astype(np.float32) + b32).astype(np.float32)

    # stage 1: group scores and the M kept groups
    score32 = _top_sum_f32(sb32.reshape(T, G, n), group_topn)               # [T, G]
    order_g = np.argsort(-score32, axis=1, kind="stable")
    groups = order_g[:, :M].astype(np.int32)
    nt_g = np.zeros(T, bool)
    if M < G:
        score64 = (-np.sort(-sb.reshape(T, G, n), axis=2))[:, :, :group_topn].sum(2)
        nt_g = _gap_at(score64, order_g, M) < NEAR_TIE

    # stage 2: top-K experts among the kept groups' experts
    kept = np.zeros((T, G), bool)
    np.put_along_axis(kept, groups.astype(np.int64), True, axis=1)
    cand = np.repeat(kept, n, axis=1)                                        # [T, E]
    masked = np.where(cand, sb32, np.float32(-np.inf))
    order_e = np.argsort(-masked, axis=1, kind="stable")
    idx = order_e[:, :K].astype(np.int32)
    nt_e = np.zeros(T, bool)
    if K < M * n:
        nt_e = _gap_at(np.where(cand, sb, -np.inf), order_e, K) < NEAR_TIE
    sel_sb = np.take_along_axis(sb, order_e[:, :K], 1)
    nt_o = np.any(np.abs(np.diff(sel_sb, axis=1)) < NEAR_TIE, axis=1) if K > 1 else np.zeros(T, bool)

    ss = np.take_along_axis(s, order_e[:, :K], 1)
    gate = ss / ss.sum(1, keepdims=True)
    return RouteResult(idx, gate, s, sb, groups, nt_g, nt_e, nt_o)


def permute(idx: np.ndarray, num_experts: int):
    """Group the (token, expert) pairs by expert, tokens ascending within an expert.

    No pair is dropped ([R] 2.4).  Returns
      load [E] int32          pairs per expert (the "whole batch" load of [R] 2.3)
      offsets [E+1] int32     exclusive prefix sum of load
      row_token [T*K] int32   token of each expert-sorted row
      pair_row [T*K] int32    row of pair (t, k), flattened t*K + k
    """
    T, K = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    load = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    offsets[1:] = np.cumsum(load)
    order = np.argsort(flat, kind="stable")          # stable: tokens ascending per expert
    row_token = (order // K).astype(np.int32)
    pair_row = np.empty(T * K, np.int32)
    pair_row[order] = np.arange(T * K, dtype=np.int32)
    return load, offsets, row_token, pair_row


def expert_ffn(u, w_gate, w_up, w_down) -> np.ndarray:
    """SwiGLU expert: W_down (silu(W_gate u) * (W_up u)) for each row u of ``u``.

    u [n, h], w_gate/w_up [inter, h], w_down [h, inter] -> [n, h] float64.
    """
    u = _f64(u)
    a = u @ _f64(w_gate).T
    v = u @ _f64(w_up).T
    return (silu(a) * v) @ _f64(w_down).T


def layer_output(x, idx, gate, get_expert, num_experts: int, num_shared: int,
                 rows=None, residual=None, ffn=expert_ffn) -> np.ndarray:
    """out_t = [u_t] + sum_s FFN_{E+s}(u_t) + sum_k g_tk FFN_{idx_tk}(u_t)   ([R] 2.2).

    get_expert(e) -> (w_gate, w_up, w_down) for expert e (routed 0..E-1, shared E..E+Ns-1);
    it is called once per expert that the compared rows touch, so large expert sets
    can be streamed.  ``rows`` selects the tokens to evaluate (default: all).
    """
    x64 = _f64(x)
    T = x64.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    u = x64[rows]
    out = np.zeros_like(u)
    for s in range(num_shared):
        out += ffn(u, *get_expert(num_experts + s))
    sel = np.asarray(idx)[rows]
    g = np.asarray(gate, dtype=np.float64)[rows]
    for e in np.unique(sel):
        r, k = np.nonzero(sel == e)
        out[r] += g[r, k][:, None] * ffn(u[r], *get_expert(int(e)))
    if residual is not None:
        out += _f64(residual)[rows]
    return out


def bias_update(load, bias, gamma: float, num_tokens: int, top_k: int) -> np.ndarray:
    """Auxiliary-loss-free bias update at the end of a step ([R] 2.3), float32 arithmetic.

    Mean load is T*K/E; compared in integers as load_e * E against T * K:
      load_e * E > T*K  (overloaded)   ->  b_e = f32(b_e - gamma)
      load_e * E < T*K  (underloaded)  ->  b_e = f32(b_e + gamma)
      equal                            ->  unchanged
    """
    load = np.asarray(load, dtype=np.int64)
    E = load.shape[0]
    b = np.asarray(bias, dtype=np.float32).copy()
    g = np.float32(gamma)
    total = np.int64(num_tokens) * np.int64(top_k)
    for e in range(E):
        if load[e] * E > total:
            b[e] = np.float32(b[e] - g)
        elif load[e] * E < total:
            b[e] = np.float32(b[e] + g)
    return b


def valid_selections(sb_t: np.ndarray, num_groups: int, top_groups: int, group_topn: int,
                     top_k: int, tol: float = NEAR_TIE) -> set:
    """Every expert set one token may legitimately select when gaps below ``tol`` are
    treated as ties ([R] 2.3-2.4 with the near-tie reading): a K-set X is valid iff
    some set S of M groups has
      min_{g in S} score_g >= max_{g not in S} score_g - tol   (S is a top-M group set)
      X within the experts of S, and
      min_{e in X} sb_e >= max_{e in S, not in X} sb_e - tol    (X is a top-K of S),
    score_g being the sum of the group_topn largest float64 sb of group g.
    sb_t [E] float64 biased affinities of the token.  Returns a set of frozensets.

    Within a top-M (top-K) set every member must be at least the (M+1)-th (K+1)-th
    value minus tol, and everything above the M-th (K-th) value plus tol is forced
    in, so only the values within tol of the boundary are enumerated."""
    import itertools
    sb_t = np.asarray(sb_t, np.float64)
    E = sb_t.shape[0]
    G, M, K = num_groups, top_groups, top_k
    n = E // G
    score = (-np.sort(-sb_t.reshape(G, n), axis=1))[:, :group_topn].sum(1)

    def top_sets(vals, keys, k):
        """All k-subsets of keys whose values form a top-k within tol."""
        order = sorted(keys, key=lambda i: -vals[i])
        if k >= len(order):
            return [frozenset(order)]
        vk = vals[order[k - 1]]
        forced = [i for i in order if vals[i] > vk + tol]
        window = [i for i in order if vk - tol <= vals[i] <= vk + tol]
        out = []
        for extra in itertools.combinations(window, k - len(forced)):
            xs = frozenset(forced) | frozenset(extra)
            rest = [vals[i] for i in keys if i not in xs]
            if not rest or min(vals[i] for i in xs) >= max(rest) - tol:
                out.append(xs)
        return out

    result = set()
    for gs in top_sets(score, list(range(G)), M):
        cand = [e for g in sorted(gs) for e in range(g * n, (g + 1) * n)]
        result.update(top_sets(sb_t, cand, K))
    return result
