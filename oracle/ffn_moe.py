"""Plain float64 definition of the MiniMind FFN sub-layer forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obvious on
purpose: library matmuls are used as steps, nothing is blocked, fused or
reordered beyond what the definition states.

Page citations:
  [L13]  MiniMind course, lesson 13 "FFN and MoE"
  [MM4]  minimind3.com, chapter 4 "MLP & MoE"
  [DEMO] minimind3.com, chapter 4 example script
  [NOTE] "MiniMind study notes 08: FeedForward and MoE"

Readings where the pages are silent or ambiguous (all listed in the design doc):
  * top-k slot order: probability descending, ties to the lower expert id
    (the pages call topk with sorted=False, which fixes no order);
  * y accumulates the selected experts in ascending expert id (the pages loop
    ``for i, expert in enumerate(self.experts)``);
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
    """Per-expert token lists ([L13] section 3 step 5: ``mask = topk_idx == i``,
    ``token_idx = mask.any(-1).nonzero()``): L_e = ascending tokens that chose e.

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


# --------------------------------------------------------------------- MoE
def moe_route(x, Wr, k, coef, norm_topk_prob=True):
    """Routing half of the MoE forward: probabilities, top-k, renormalised
    (or, with norm_topk_prob False, raw) weights, per-expert lists and
    aux_loss ([L13] section 3 steps 4-6)."""
    p = router_probs(x, Wr)
    E = p.shape[1]
    idx = topk_canonical(p, k)
    alpha = renorm_weights(p, idx, normalize=norm_topk_prob)
    counts, offsets, sorted_ids = expert_lists(idx, E)
    return {
        "p": p,
        "topk_idx": idx,
        "alpha": alpha,
        "counts": counts,
        "offsets": offsets,
        "sorted_token_ids": sorted_ids,
        "aux": aux_loss(p, idx, E, coef),
    }


def moe_ffn(x, Wr, Wg, Wu, Wd, k, coef, rows=None, route=None, residual=None,
            norm_topk_prob=True):
    """MoE FFN forward ([L13] section 0 MoE equations, section 3 steps 4-6;
    [MM4] 4.3 steps 1-3):

        y_t = sum over e in S_t, ascending e, of alpha_{t,e} * Expert_e(x_t),

    starting from zeros, each expert applied only to the tokens that chose it
    (gather its rows, run the expert, scale, add back into their rows).

    x [N, H]; Wr [E, H]; Wg, Wu [E, I, H]; Wd [E, H, I].  ``rows`` (sorted or
    not) restricts y to those tokens; routing statistics always use all N.
    ``residual`` [N, H] (optional) starts y from the residual stream instead of
    zeros ([L13] section 1.3 and 1.4: hidden_states + mlp(...)).
    Returns the routing dict plus ``y`` ([len(rows), H] or [N, H]).
    """
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    r = moe_route(x, Wr, k, coef, norm_topk_prob) if route is None else route
    idx, alpha = r["topk_idx"], r["alpha"]
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
        mask = idx == e                                  # [N, k]
        tok = np.nonzero(mask.any(axis=1))[0]            # ascending tokens that chose e
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
