"""Plain float64 definition of the MiniMind FFN sub-layer forward pass and its
gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obvious on
purpose: library matmuls are used as steps, nothing is blocked, fused or
reordered beyond what the definition states.

Page citations:
  [L13]  MiniMind course, lesson 13 "FFN and MoE"
  [MM4]  minimind3.com, chapter 4 "MLP & MoE"
  [DEMO] minimind3.com, chapter 4 example script
  [NOTE] "MiniMind study notes 08: FeedForward and MoE"

Readings where the pages are silent or ambiguous:
  * top-k slot order: probability descending, ties to the lower expert id
    (the pages call topk with sorted=False, which fixes no order);
  * y accumulates the selected experts in ascending expert id (the pages' module
    visits the experts in index order);
  * aux for k > 1 keeps the one-hot load as [k, E] and broadcasts, exactly as
    the module code does, so uniform routing gives k * coef.
"""
from __future__ import annotations

import numpy as np

EPS_RENORM = 1e-20  # [L13] section 3 step 5 / [MM4] 4.3 step 2: added to the top-k sum


# --------------------------------------------------------------------- SiLU
def silu(z):
    """SiLU(z) = z * sigmoid(z)  ([MM4] 4.2 "silu(x) = x * sigmoid(x)").

    For z < 0 the equivalent z * e^z / (1 + e^z) avoids overflow of e^{-z}.
    """
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    zp = z[pos]
    out[pos] = zp / (1.0 + np.exp(-zp))
    zn = z[~pos]
    ez = np.exp(zn)
    out[~pos] = zn * ez / (1.0 + ez)
    return out


# ---------------------------------------------------------------- dense FFN
def swiglu_ffn(x, Wg, Wu, Wd):
    """Dense SwiGLU FFN on token rows ([L13] section 0 and 1.2 equations;
    section 3 step 3):  g = Wg x, u = Wu x, h = SiLU(g) * u, y = Wd h.

    x [T, H]; Wg, Wu [I, H]; Wd [H, I] (nn.Linear [out, in]).  Returns y [T, H].
    """
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(Wg, dtype=np.float64).T   # [T, I]
    u = x @ np.asarray(Wu, dtype=np.float64).T   # [T, I]
    h = silu(g) * u                              # [T, I]
    return h @ np.asarray(Wd, dtype=np.float64).T  # [T, H]


def dense_ffn(x, Wg, Wu, Wd, rows=None, residual=None):
    """Dense FFN forward; ``rows`` restricts the output to those token rows
    (each token is transformed independently, [L13] section 1.1).

    ``residual`` [N, H] (optional): the block's residual stream, returned as
    residual + FFN(x) ([L13] section 1.3: hidden_states + mlp(...)).
    """
    x = np.asarray(x, dtype=np.float64)
    if rows is not None:
        x = x[np.asarray(rows)]
    y = swiglu_ffn(x, Wg, Wu, Wd)
    if residual is not None:
        r = np.asarray(residual, dtype=np.float64)
        y = (r[np.asarray(rows)] if rows is not None else r) + y
    return y


# ------------------------------------------------------------------ router
def router_probs(x, Wr):
    """p = softmax(Wr x) per token ([L13] section 1.5, router equations).

    The max logit is subtracted first; the quotient is mathematically identical
    to exp(r_e) / sum_j exp(r_j).  x [N, H], Wr [E, H] -> p [N, E].
    """
    r = np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T
    r = r - r.max(axis=1, keepdims=True)
    ex = np.exp(r)
    return ex / ex.sum(axis=1, keepdims=True)


def topk_canonical(p, k):
    """S_t = TopK(p_t, k) ([L13] section 0 MoE equations, section 3 step 4).

    Slot order: probability descending, equal probabilities by ascending expert
    id (a stable sort of -p).  Returns int64 [N, k].
    """
    p = np.asarray(p, dtype=np.float64)
    order = np.argsort(-p, axis=1, kind="stable")
    return order[:, :k].copy()


def renorm_weights(p, idx, normalize=True):
    """alpha_{t,j} = p_{t,S_j} / (sum_{j'} p_{t,S_j'} + 1e-20)
    ([L13] section 0 alpha equation; section 3 step 5 norm_topk_prob line).

    normalize=False is the config's norm_topk_prob = False branch ([L13]
    section 3 step 1 config, step 5): the selected probabilities as they are.
    """
    p = np.asarray(p, dtype=np.float64)
    ps = np.take_along_axis(p, np.asarray(idx), axis=1)
    if not normalize:
        return ps
    return ps / (ps.sum(axis=1, keepdims=True) + EPS_RENORM)


def expert_lists(idx, E):
    """Per-expert token lists ([L13] section 3 step 5: a token belongs to expert
    e's list when e is among its selections; the list is in token order):
    L_e = ascending tokens that chose e.

    Returns counts [E], offsets [E+1] (exclusive prefix sum) and
    sorted_token_ids = concatenation of L_0, ..., L_{E-1}.
    """
    idx = np.asarray(idx)
    lists = [np.nonzero((idx == e).any(axis=1))[0] for e in range(E)]
    counts = np.array([len(L) for L in lists], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_ids = np.concatenate(lists) if lists else np.zeros(0, np.int64)
    return counts, offsets, sorted_ids.astype(np.int64)


def aux_loss(p, idx, E, coef):
    """Load-balancing loss ([L13] section 1.6 equation and section 3 step 6;
    [MM4] 4.4):  load = one_hot(idx, E).mean(0)  -> [k, E];
    prob = p.mean(0) -> [E];  aux = sum(load * prob) * E * coef.

    coef == 0 reproduces the disabled branch (a zero scalar).
    """
    if coef == 0.0:
        return 0.0
    p = np.asarray(p, dtype=np.float64)
    idx = np.asarray(idx)
    N, K = idx.shape
    one_hot = np.zeros((N, K, E))
    for j in range(K):
        one_hot[np.arange(N), j, idx[:, j]] = 1.0
    load = one_hot.mean(axis=0)     # [K, E]
    prob = p.mean(axis=0)           # [E]
    return float((load * prob[None, :]).sum() * E * coef)


# ------------------------------------------------- z-loss and capacity
# The study notes' section 10 table names both (z-loss keeps the router
# logits from growing; capacity limits how many tokens one expert takes) and
# lesson 13 section 4 lists capacity / token dropping as not required; no
# page defines them.  These follow the standard published forms (readings,
# listed with the design notes):
#   z-loss    z_coef * mean_t (logsumexp_e r_te)^2
#   capacity  C = ceil(capacity_factor * N * k / E) (capacity_factor 0: no
#             limit); expert e keeps the first C of its tokens in the
#             dispatch order (ascending token id) and drops the rest; a
#             dropped (token, expert) pair adds nothing to y; alpha is not
#             renormalised; aux uses the router's choices before dropping.
def logsumexp_rows(r):
    """log sum_e exp(r_te) per row, shifted by the row maximum (no overflow)."""
    r = np.asarray(r, dtype=np.float64)
    m = r.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(r - m).sum(axis=1, keepdims=True)))[:, 0]


def router_z_loss(x, Wr, z_coef):
    """z_coef * mean over tokens of logsumexp(W_r x_t)^2 (0 when z_coef is 0)."""
    if z_coef == 0.0:
        return 0.0
    r = np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T
    return float(z_coef * np.mean(logsumexp_rows(r) ** 2))


def expert_capacity(N, k, E, capacity_factor):
    """C = ceil(capacity_factor * N * k / E); None for capacity_factor 0 (no limit)."""
    if capacity_factor == 0.0:
        return None
    return int(np.ceil(capacity_factor * N * k / E))


def kept_entries(idx, E, C):
    """keep [N, k]: True where (token, slot) is among the first C tokens of its
    expert in ascending token order (all True when C is None)."""
    idx = np.asarray(idx)
    keep = np.ones(idx.shape, dtype=bool)
    if C is None:
        return keep
    for e in range(E):
        t, j = np.nonzero(idx == e)          # row-major: ascending token
        keep[t[C:], j[C:]] = False
    return keep


# --------------------------------------------------------------------- MoE
def moe_route(x, Wr, k, coef, norm_topk_prob=True, z_coef=0.0, capacity_factor=0.0):
    """Routing half of the MoE forward: probabilities, top-k, renormalised
    (or, with norm_topk_prob False, raw) weights, per-expert lists and
    aux_loss ([L13] section 3 steps 4-6); with the readings above also the
    z-loss and, under a capacity, the kept entries, their per-expert counts,
    offsets and token lists (the plain lists and aux stay pre-drop)."""
    p = router_probs(x, Wr)
    E = p.shape[1]
    N = p.shape[0]
    idx = topk_canonical(p, k)
    alpha = renorm_weights(p, idx, normalize=norm_topk_prob)
    counts, offsets, sorted_ids = expert_lists(idx, E)
    C = expert_capacity(N, k, E, capacity_factor)
    keep = kept_entries(idx, E, C)
    kept_counts = np.array([int(keep[idx == e].sum()) for e in range(E)], dtype=np.int64)
    kept_offsets = np.zeros(E + 1, dtype=np.int64)
    kept_offsets[1:] = np.cumsum(kept_counts)
    kept_ids = [np.nonzero(((idx == e) & keep).any(axis=1))[0] for e in range(E)]
    kept_sorted = np.concatenate(kept_ids) if kept_ids else np.zeros(0, np.int64)
    return {
        "p": p,
        "topk_idx": idx,
        "alpha": alpha,
        "counts": counts,
        "offsets": offsets,
        "sorted_token_ids": sorted_ids,
        "aux": aux_loss(p, idx, E, coef),
        "z_loss": router_z_loss(x, Wr, z_coef),
        "capacity": C,
        "keep": keep,
        "kept_counts": kept_counts,
        "kept_offsets": kept_offsets,
        "kept_sorted_token_ids": kept_sorted.astype(np.int64),
    }


def moe_ffn(x, Wr, Wg, Wu, Wd, k, coef, rows=None, route=None, residual=None,
            norm_topk_prob=True, z_coef=0.0, capacity_factor=0.0):
    """MoE FFN forward ([L13] section 0 MoE equations, section 3 steps 4-6;
    [MM4] 4.3 steps 1-3):

        y_t = sum over e in S_t, ascending e, of alpha_{t,e} * Expert_e(x_t),

    starting from zeros, each expert applied only to the tokens that chose it
    (gather its rows, run the expert, scale, add back into their rows).

    x [N, H]; Wr [E, H]; Wg, Wu [E, I, H]; Wd [E, H, I].  ``rows`` (sorted or
    not) restricts y to those tokens; routing statistics always use all N.
    ``residual`` [N, H] (optional) starts y from the residual stream instead of
    zeros ([L13] section 1.3 and 1.4: hidden_states + mlp(...)).  Under a
    capacity only the kept (token, expert) pairs contribute.
    Returns the routing dict plus ``y`` ([len(rows), H] or [N, H]).
    """
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    r = (moe_route(x, Wr, k, coef, norm_topk_prob, z_coef, capacity_factor) if route is None
         else route)
    idx, alpha = r["topk_idx"], r["alpha"]
    keep = r.get("keep", np.ones(np.shape(idx), dtype=bool))
    E = r["p"].shape[1]
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows, dtype=np.int64)
    where = -np.ones(N, dtype=np.int64)
    where[rows] = np.arange(len(rows))
    if residual is None:
        y = np.zeros((len(rows), x.shape[1]))
    else:
        y = np.asarray(residual, dtype=np.float64)[rows].copy()
    for e in range(E):
        mask = (idx == e) & keep                         # [N, k]
        tok = np.nonzero(mask.any(axis=1))[0]            # ascending kept tokens that chose e
        tok = tok[where[tok] >= 0]
        if tok.size == 0:
            continue
        w = alpha[tok][mask[tok]]                        # one weight per token (distinct experts per token)
        out = swiglu_ffn(x[tok], Wg[e], Wu[e], Wd[e])
        y[where[tok]] += w[:, None] * out
    res = dict(r)
    res["y"] = y
    res["rows"] = rows
    return res


# ----------------------------------------------------------------- backward
# Gradients of the forward above with respect to its inputs and weights, the
# ones autograd gives: the top-k selection and the per-expert counts are
# discrete and carry no gradient; the selected weights (from the softmax) and
# the mean probabilities in aux carry it back to the router ([NOTES] section 7
# "how the router is trained"; [MM4] 4.4: f_i is not differentiable, P_i is).
def silu_grad(z):
    """d SiLU / dz = sigma(z) * (1 + z * (1 - sigma(z)))  (derivative of the
    [MM4] 4.2 definition z * sigmoid(z)); overflow-safe sigma."""
    z = np.asarray(z, dtype=np.float64)
    s = np.empty_like(z)
    pos = z >= 0
    s[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    s[~pos] = ez / (1.0 + ez)
    return s * (1.0 + z * (1.0 - s))


def swiglu_ffn_bwd(x, Wg, Wu, Wd, dy):
    """Backward of ``swiglu_ffn`` for upstream dy [T, H]: returns dx [T, H],
    dWg [I, H], dWu [I, H], dWd [H, I].

    Chain rule through g = Wg x, u = Wu x, h = SiLU(g) u, y = Wd h.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    Wg, Wu, Wd = (np.asarray(a, dtype=np.float64) for a in (Wg, Wu, Wd))
    g = x @ Wg.T
    u = x @ Wu.T
    s = silu(g)
    h = s * u
    dWd = dy.T @ h                    # [H, I]
    dh = dy @ Wd                      # [T, I]
    dg = dh * u * silu_grad(g)
    du = dh * s
    dWg = dg.T @ x                    # [I, H]
    dWu = du.T @ x
    dx = dg @ Wg + du @ Wu            # [T, H]
    return dx, dWg, dWu, dWd


def moe_ffn_bwd(x, Wr, Wg, Wu, Wd, k, coef, dy, daux=1.0, norm_topk_prob=True,
                z_coef=0.0, dz=1.0, capacity_factor=0.0):
    """Backward of ``moe_ffn`` (with its aux_loss) for upstream dy [N, H] and
    daux (the gradient reaching aux_loss; 1 when it is added to the loss).

    Returns dict dx [N, H], dWr [E, H], dWg / dWu [E, I, H], dWd [E, H, I] and
    the forward's routing.  Per expert e and token t with e in S_t:
      o = Expert_e(x_t), y_t += alpha_{t,e} o   =>  d alpha_{t,e} = dy_t . o,
      the expert's own backward with upstream alpha_{t,e} dy_t;
    then through alpha = p_S / (sum p_S + 1e-20) (or alpha = p_S), the aux term
    coef * E * sum_e c_e * (sum_t p_te) / N^2 (counts constant), the softmax
    and the router logits r = Wr x.  The z-loss z_coef * mean_t lse_t^2 (with
    upstream dz) adds z_coef * dz * 2 lse_t p_te / N to d r_te (d lse / d r = p);
    a pair dropped by the capacity passes nothing (no expert gradient, d alpha 0).
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    Wr = np.asarray(Wr, dtype=np.float64)
    N, H = x.shape
    E = Wr.shape[0]
    r = moe_route(x, Wr, k, coef, norm_topk_prob, z_coef, capacity_factor)
    p, idx, alpha, counts = r["p"], r["topk_idx"], r["alpha"], r["counts"]
    keep = r["keep"]
    dx = np.zeros_like(x)
    dWg = np.zeros(np.shape(Wg))
    dWu = np.zeros(np.shape(Wu))
    dWd = np.zeros(np.shape(Wd))
    dalpha = np.zeros(alpha.shape)
    for e in range(E):
        mask = (idx == e) & keep
        tok = np.nonzero(mask.any(axis=1))[0]
        if tok.size == 0:
            continue
        slot = np.argmax(mask[tok], axis=1)               # which of the k slots holds e
        w = alpha[tok, slot]
        o = swiglu_ffn(x[tok], Wg[e], Wu[e], Wd[e])
        dalpha[tok, slot] = (dy[tok] * o).sum(axis=1)
        gx, gWg, gWu, gWd = swiglu_ffn_bwd(x[tok], Wg[e], Wu[e], Wd[e], w[:, None] * dy[tok])
        dx[tok] += gx
        dWg[e] += gWg
        dWu[e] += gWu
        dWd[e] += gWd
    # selected weights -> probabilities
    ps = np.take_along_axis(p, idx, axis=1)
    dp = np.zeros_like(p)
    if norm_topk_prob:
        Z = ps.sum(axis=1, keepdims=True) + EPS_RENORM
        dps = dalpha / Z - (dalpha * ps).sum(axis=1, keepdims=True) / Z ** 2
    else:
        dps = dalpha
    np.put_along_axis(dp, idx, dps, axis=1)
    # aux = coef * E * sum_e c_e * sum_t p_te / N^2  (c_e constant)
    if coef != 0.0:
        dp += daux * coef * E * counts[None, :] / float(N) ** 2
    # softmax and router logits
    dr = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    if z_coef != 0.0:
        lse = logsumexp_rows(x @ Wr.T)
        dr += (z_coef * dz * 2.0 / N) * lse[:, None] * p
    dWr = dr.T @ x
    dx += dr @ Wr
    return {"dx": dx, "dWr": dWr, "dWg": dWg, "dWu": dWu, "dWd": dWd, "route": r}


def moe_ffn_bwd_sampled(x, Wr, Wg, Wu, Wd, k, coef, dy, daux=1.0, norm_topk_prob=True,
                        rows=None, units=None, z_coef=0.0, dz=1.0, capacity_factor=0.0):
    """Exact parts of ``moe_ffn_bwd`` at a fraction of its cost, for checks at
    full size.

    * dx[rows]: each token's input gradient needs only its own selected
      experts (their outputs for that token give d alpha), the routing counts
      (aux term) and the router weights, so it is computed row by row.
    * dWg[e][units], dWu[e][units], dWd[e][:, units]: the FFN is a sum over its
      intermediate units, and a unit's weight gradients involve only that
      unit's g, u and down column, so the expert backward restricted to those
      units (upstream alpha * dy over all the expert's tokens) gives them
      exactly.

    * dW_r (only when every row is taken): the sum of dr_t x_t^T over them.

    Returns dict dx_rows [len(rows), H], rows, units, dWg_u / dWu_u
    [E, len(units), H], dWd_u [E, H, len(units)], dWr (or None) and the routing.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    Wr = np.asarray(Wr, dtype=np.float64)
    N, H = x.shape
    E = Wr.shape[0]
    r = moe_route(x, Wr, k, coef, norm_topk_prob, z_coef, capacity_factor)
    p, idx, alpha, counts = r["p"], r["topk_idx"], r["alpha"], r["counts"]
    keep = r["keep"]
    lse = logsumexp_rows(x @ Wr.T) if z_coef != 0.0 else None
    all_rows = rows is None
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    units = np.arange(np.shape(Wg)[1]) if units is None else np.asarray(units, dtype=np.int64)
    # dx for the sampled rows
    dx = np.zeros((len(rows), H))
    drs = np.zeros((len(rows), E))
    for n, t in enumerate(rows):
        dalpha = np.zeros(k)
        for j in range(k):
            if not keep[t, j]:
                continue
            e = idx[t, j]
            xt = x[t:t + 1]
            o = swiglu_ffn(xt, Wg[e], Wu[e], Wd[e])[0]
            dalpha[j] = dy[t] @ o
            gx = swiglu_ffn_bwd(xt, Wg[e], Wu[e], Wd[e], alpha[t, j] * dy[t:t + 1])[0]
            dx[n] += gx[0]
        ps = p[t, idx[t]]
        if norm_topk_prob:
            Z = ps.sum() + EPS_RENORM
            dps = dalpha / Z - (dalpha * ps).sum() / Z ** 2
        else:
            dps = dalpha
        dp = np.zeros(E)
        dp[idx[t]] = dps
        if coef != 0.0:
            dp += daux * coef * E * counts / float(N) ** 2
        dr = p[t] * (dp - (p[t] * dp).sum())
        if lse is not None:
            dr = dr + (z_coef * dz * 2.0 / N) * lse[t] * p[t]
        drs[n] = dr
        dx[n] += dr @ Wr
    # weight gradients of the sampled units
    dWg_u = np.zeros((E, len(units), H))
    dWu_u = np.zeros((E, len(units), H))
    dWd_u = np.zeros((E, H, len(units)))
    for e in range(E):
        mask = (idx == e) & keep
        tok = np.nonzero(mask.any(axis=1))[0]
        if tok.size == 0:
            continue
        slot = np.argmax(mask[tok], axis=1)
        w = alpha[tok, slot]
        _, gWg, gWu, gWd = swiglu_ffn_bwd(x[tok], np.asarray(Wg[e])[units], np.asarray(Wu[e])[units],
                                          np.asarray(Wd[e])[:, units], w[:, None] * dy[tok])
        dWg_u[e], dWu_u[e], dWd_u[e] = gWg, gWu, gWd
    return {"dx_rows": dx, "rows": rows, "units": units, "dWg_u": dWg_u, "dWu_u": dWu_u,
            "dWd_u": dWd_u, "dWr": drs.T @ x if all_rows else None, "route": r}
