"""MoE feed-forward layer with int8 expert weights, oracle side (test infrastructure).

Sources (Jamba-1.5 paper):
  * "Model Architecture": the MLP is replaced by an MoE module every e=2
    layers; n=16 experts; the top K=2 are selected for each token.
  * "Serving Considerations and Improvements": ExpertsInt8 -- expert weights
    are int8 in memory and are turned back into BF16 values inside the fused
    MoE kernel; activations stay BF16.
Jamba paper summary (Lieber et al. 2024, "Key points"): 16 experts, two per
token, MoE every other layer.

Readings where the pages are silent:
  * gate: p = softmax over all E logits; the K experts with the largest
    logits, in descending order, exact ties to the lower expert index;
    weights w_k = p_k / sum_j p_j over the K chosen experts;
  * expert: SwiGLU, o = s_d * (q_d @ h) with h = silu(g) * u,
    g = s_g * (q_g @ x), u = s_u * (q_u @ x), silu(z) = z / (1 + exp(-z));
  * combine: y_t = sum_k w_k * o_{t,k}; no capacity limit, nothing dropped,
    no residual, no normalisation.
Everything is fp64 on exact copies of the inputs. Weight layout is (out, in):
q_g, q_u [E, f, d], q_d [E, d, f]; scales s_g, s_u [E, f], s_d [E, d];
router_w [E, d].
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- router
def router_logits(x, router_w, bias=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * router_w[e, i] (+ bias[e]); fp64 [T, E]."""
    l = _f64(x) @ _f64(router_w).T
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l


def softmax(l) -> np.ndarray:
    l = _f64(l)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def topk_gate(logits, K: int):
    """Top-K selection and renormalised gate weights.

    Returns ids int32 [T, K] (descending logit; exact ties to the lower index)
    and w fp64 [T, K] with w[t, k] = p[t, ids[t,k]] / sum_j p[t, ids[t,j]].
    """
    l = _f64(logits)
    T, E = l.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    # a stable sort of -l keeps equal logits in ascending expert order
    order = np.argsort(-l, axis=1, kind="stable")
    ids = order[:, :K].astype(np.int32)
    p = softmax(l)
    pk = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = pk / pk.sum(axis=1, keepdims=True)
    return ids, w


def near_tie_flags(logits, K: int, gap: float = 1e-4) -> np.ndarray:
    """Tokens whose top-K selection is fragile under rounding of the logits.

    Flag t when two neighbouring order statistics among the first K+1 sorted
    logits are closer than `gap`: the order inside the selection, or the
    membership of the selection, may then legitimately differ.
    """
    l = np.sort(_f64(logits), axis=1)[:, ::-1]
    E = l.shape[1]
    m = min(K + 1, E)
    if m < 2:
        return np.zeros(l.shape[0], dtype=bool)
    d = l[:, : m - 1] - l[:, 1:m]
    return np.any(d < gap, axis=1)


def route(x, router_w, bias, K: int):
    """Router + gate: (ids [T,K] int32, w [T,K] fp64, logits [T,E] fp64)."""
    l = router_logits(x, router_w, bias)
    ids, w = topk_gate(l, K)
    return ids, w, l


# --------------------------------------------------------------------------- permute
def permute(ids, E: int):
    """Group the T*K slots by expert.

    Slot s = t*K + k carries expert ids[t, k]. Returns
      offsets      int32 [E+1]: expert e owns sorted rows [offsets[e], offsets[e+1]),
      sorted_slots int32 [T*K]: slot held by each sorted row, ascending within an expert,
      slot_to_row  int32 [T*K]: inverse map, sorted row of each slot.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_slots = np.argsort(flat, kind="stable")
    slot_to_row = np.empty_like(sorted_slots)
    slot_to_row[sorted_slots] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_slots.astype(np.int32), slot_to_row.astype(np.int32)


# --------------------------------------------------------------------------- experts
def silu(z) -> np.ndarray:
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def expert_hidden(xrows, q_gate, s_gate, q_up, s_up) -> np.ndarray:
    """The gated hidden activation of one expert: xrows [n, d] -> h [n, c], fp64.

    g = s_g * (x @ q_g^T), u = s_u * (x @ q_u^T), h = silu(g) * u, for the c
    output channels (rows) of q_gate / q_up given; each channel of h depends
    only on its own row of each matrix, so any subset of channels may be passed.
    """
    x = _f64(xrows)
    g = (x @ _f64(q_gate).T) * _f64(s_gate)[None, :]
    u = (x @ _f64(q_up).T) * _f64(s_up)[None, :]
    return silu(g) * u


def expert_swiglu(xrows, q_gate, s_gate, q_up, s_up, q_down, s_down) -> np.ndarray:
    """One expert on a block of rows: xrows [n, d] -> [n, d], fp64.

    h = expert_hidden(x) over all f channels, o = s_d * (h @ q_d^T). Scales are
    per output channel, so they multiply the columns of each product.
    """
    h = expert_hidden(xrows, q_gate, s_gate, q_up, s_up)
    return (h @ _f64(q_down).T) * _f64(s_down)[None, :]


def expert_outputs(x, ids, weights: dict, experts=None) -> np.ndarray:
    """Per-slot expert outputs o [T, K, d] (fp64) for the given routing.

    `weights` holds q_gate, s_gate, q_up, s_up, q_down, s_down (whole [E, ...]
    arrays, or dicts e -> per-expert arrays). Only slots whose expert is in
    `experts` (default: all) are computed; the others stay NaN.
    """
    x = _f64(x)
    ids = np.asarray(ids)
    T, K = ids.shape
    d = x.shape[1]
    o = np.full((T, K, d), np.nan)
    touched = np.unique(ids) if experts is None else np.asarray(sorted(experts))
    for e in touched:
        tt, kk = np.nonzero(ids == e)
        if tt.size == 0:
            continue
        o[tt, kk] = expert_swiglu(
            x[tt], weights["q_gate"][e], weights["s_gate"][e], weights["q_up"][e],
            weights["s_up"][e], weights["q_down"][e], weights["s_down"][e])
    return o


def combine(o, w) -> np.ndarray:
    """y[t] = sum_k w[t, k] * o[t, k]  (k ascending), fp64 [T, d]."""
    o = _f64(o)
    w = _f64(w)
    y = np.zeros((o.shape[0], o.shape[2]))
    for k in range(o.shape[1]):
        y += w[:, k, None] * o[:, k]
    return y


def moe_forward(x, router_w, bias, weights: dict, K: int, ids=None):
    """The whole layer. Returns dict(y, ids, w, logits).

    With `ids` given, routing is forced to those experts (the gate weights are
    still the renormalised softmax of the router logits over them).
    """
    logits = router_logits(x, router_w, bias)
    if ids is None:
        ids, w = topk_gate(logits, K)
    else:
        ids = np.asarray(ids, dtype=np.int32)
        p = softmax(logits)
        pk = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        w = pk / pk.sum(axis=1, keepdims=True)
    o = expert_outputs(x, ids, weights)
    return {"y": combine(o, w), "ids": ids, "w": w, "logits": logits}


def dense_mixture(x, router_w, bias, weights: dict) -> np.ndarray:
    """sum_e softmax(l)_e * FFN_e(x) over every expert (the K = E case)."""
    x = _f64(x)
    p = softmax(router_logits(x, router_w, bias))
    E = p.shape[1]
    y = np.zeros_like(x)
    for e in range(E):
        y += p[:, e, None] * expert_swiglu(
            x, weights["q_gate"][e], weights["s_gate"][e], weights["q_up"][e],
            weights["s_up"][e], weights["q_down"][e], weights["s_down"][e])
    return y


def moe_forward_loop(x, router_w, bias, weights: dict, K: int) -> np.ndarray:
    """Token-by-token statement of the layer with scalar Python loops (tiny inputs only)."""
    import math
    x = _f64(x)
    Wr = _f64(router_w)
    T, d = x.shape
    E = Wr.shape[0]
    y = np.zeros((T, d))
    for t in range(T):
        l = [sum(x[t, i] * Wr[e, i] for i in range(d)) + (0.0 if bias is None else float(bias[e]))
             for e in range(E)]
        chosen = sorted(range(E), key=lambda e: (-l[e], e))[:K]
        mx = max(l)
        z = [math.exp(v - mx) for v in l]
        den = sum(z[e] for e in chosen)
        for e in chosen:
            qg, sg = weights["q_gate"][e], weights["s_gate"][e]
            qu, su = weights["q_up"][e], weights["s_up"][e]
            qd, sd = weights["q_down"][e], weights["s_down"][e]
            f = qg.shape[0]
            h = []
            for c in range(f):
                g = float(sg[c]) * sum(int(qg[c, i]) * x[t, i] for i in range(d))
                u = float(su[c]) * sum(int(qu[c, i]) * x[t, i] for i in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for j in range(d):
                o = float(sd[j]) * sum(int(qd[j, c]) * h[c] for c in range(f))
                y[t, j] += (z[e] / den) * o
    return y
