"""Oracle of one Medusa draft-and-verify step, in float64.

Stages, in the order the summary page ("Medusa: Simple LLM Inference
Acceleration Framework with Multiple Decoding Heads", section 3.2, information
flow steps 1-6) describes them:

1. ``medusa_heads``  -- section "MEDUSA Heads": head k's logits are
   W2_k (SiLU(W1_k h) + h); the LM head's logits are W_lm h.  No biases (the
   head equation has none).  Weights are stored [out][in]: row v of W2_k is the
   weight vector of vocabulary entry v.
2. ``topk`` / ``tree_expand`` -- "Tree Attention" steps 1-2: top-s_k per head;
   the root carries the LM head's top token; a depth-l node carries the
   rank-r_l candidate of head l.  Candidates are ordered by logit descending;
   equal logits by smaller vocabulary index.
3. ``tree_attention`` -- "Tree Attention" steps 3-5: every node attends to all
   prefix keys and to its ancestors-or-self; position id = prefix length +
   depth; rotary embedding (half-split pairs, base theta) is applied to the
   tree's queries and keys at those positions; scores are scaled by 1/sqrt(Dh).
4. ``verify_logits`` -- step 6 / "Notes on Medusa" section 3: the node outputs
   (heads concatenated) go through the LM head; per row the argmax, and at
   temperature tau > 0 the log-partition and entropy (nats) of softmax(z/tau).
5. ``accept_path`` -- "Typical Acceptance Scheme": greedy accepts a child iff
   its token is the verifier argmax at its parent; typical accepts iff
   p(x) > min(eps, delta * exp(-H(p))); at tau = 0 the verifier distribution
   is one-hot at the argmax.  The root (LM-head top token) is always accepted;
   a node is accepted iff every node on its root path passes; the result is
   the deepest accepted node (equal depth: smaller packed index).
6. ``kv_compact`` -- "MEDUSA 精读" sections 3 and 6: only the accepted path's
   keys/values stay in the cache, appended after the prefix.

Storage points: where the library's interface stores a bf16 value (the node
outputs ``o`` and the rotated tree keys ``k_rot``), the oracle rounds its
float64 value to bf16 (nearest, ties to even).  Everything else stays float64.
"""

from __future__ import annotations

import math
from typing import Dict, List

import numpy as np

from .tree import OracleTree, ancestors


# ----------------------------------------------------------------------------
# bf16 storage format (own implementation; shares nothing with the generator)
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns: they are the top 16 bits of a float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    # bf16 keeps 7 explicit mantissa bits; float64 has 52, so drop the low 45.
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    r = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


# ----------------------------------------------------------------------------
# 1. heads
# ----------------------------------------------------------------------------

def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def medusa_heads(h, W1, W2, Wlm):
    """logits[b][0] = W_lm h_b; logits[b][k] = W2_k (SiLU(W1_k h_b) + h_b), k = 1..K.

    Returns (logits [B][K+1][V] float64, a [B][K][d] float64).
    """
    hb = to_f64(h)
    B, d = hb.shape
    K = W1.shape[0]
    V = Wlm.shape[0]
    logits = np.empty((B, K + 1, V))
    a = np.empty((B, K, d))
    # every sequence's vector is multiplied by the same weights: one matrix product per weight
    logits[:, 0] = (to_f64(Wlm) @ hb.T).T
    for k in range(K):
        a[:, k] = silu((to_f64(W1[k]) @ hb.T).T) + hb
        logits[:, 1 + k] = (to_f64(W2[k]) @ a[:, k].T).T
    return logits, a


# ----------------------------------------------------------------------------
# 2. top-k and tree expansion
# ----------------------------------------------------------------------------

def topk(row: np.ndarray, k: int):
    """Indices and values of the k largest entries: value descending, then index ascending."""
    order = np.lexsort((np.arange(row.shape[0]), -row))[:k]
    return order.astype(np.int64), row[order]


def tree_expand(topk_idx: np.ndarray, tree: OracleTree, prefix_len: np.ndarray):
    """tokens[b][i] = head depth(i)'s rank(i) candidate (root: LM head top-1); pos = L_b + depth."""
    B = topk_idx.shape[0]
    T = tree.T
    tokens = np.empty((B, T), dtype=np.int64)
    pos = np.empty((B, T), dtype=np.int64)
    for b in range(B):
        for i in range(T):
            tokens[b, i] = topk_idx[b, tree.depth[i], tree.rank[i]]
            pos[b, i] = int(prefix_len[b]) + tree.depth[i]
    return tokens, pos


# ----------------------------------------------------------------------------
# 3. tree attention
# ----------------------------------------------------------------------------

def rope(x: np.ndarray, pos: int, theta: float = 10000.0) -> np.ndarray:
    """Rotary embedding, half-split pairs: (x_m, x_{m+Dh/2}) rotated by pos * theta**(-2m/Dh)."""
    Dh = x.shape[-1]
    half = Dh // 2
    m = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * m / Dh)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x, dtype=np.float64)
    out[..., :half] = x[..., :half] * c - x[..., half:] * s
    out[..., half:] = x[..., half:] * c + x[..., :half] * s
    return out


def cache_rows(Kc, Vc, b: int, L: int, page_table=None, page_size: int = 16):
    """Prefix keys/values of sequence b as [L][H][Dh] float64 (contiguous or paged)."""
    if page_table is None:
        return to_f64(Kc[b, :L]), to_f64(Vc[b, :L])
    slots = np.arange(L)
    pages = page_table[b, slots // page_size]
    return to_f64(Kc[pages, slots % page_size]), to_f64(Vc[pages, slots % page_size])


def tree_attention(q, k, v, Kc, Vc, prefix_len, tree: OracleTree, theta=10000.0,
                   bf16_store=True, page_table=None, page_size=16, heads=None, queries=None):
    """Node outputs o [B][T][H][Dh] and rotated tree keys k_rot [B][T][H][Dh].

    For every (b, h, i) the allowed keys are the L_b prefix keys followed by the
    rotated keys of i's ancestors-or-self; softmax over exactly those keys.
    ``heads`` / ``queries`` optionally restrict which (h, i) are computed (the
    others are left NaN); used to sample full-size workloads.
    """
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    B, T, H, Dh = qf.shape
    store = round_bf16 if bf16_store else (lambda x: x)
    scale = 1.0 / math.sqrt(Dh)
    k_rot = np.empty_like(kf)
    q_rot = np.empty_like(qf)
    for b in range(B):
        L = int(prefix_len[b])
        for i in range(T):
            k_rot[b, i] = store(rope(kf[b, i], L + tree.depth[i], theta))
            q_rot[b, i] = rope(qf[b, i], L + tree.depth[i], theta)
    allowed = np.zeros((T, T), dtype=bool)
    for i in range(T):
        allowed[i, ancestors(tree, i)] = True
    qs = np.arange(T) if queries is None else np.asarray(queries)
    o = np.full((B, T, H, Dh), np.nan)
    for b in range(B):
        L = int(prefix_len[b])
        pk, pv = cache_rows(Kc, Vc, b, L, page_table, page_size)
        for h in (range(H) if heads is None else heads):
            s_pre = (q_rot[b, qs, h] @ pk[:, h].T) * scale           # [nq][L]
            s_tree = (q_rot[b, qs, h] @ k_rot[b, :, h].T) * scale    # [nq][T]
            s_tree = np.where(allowed[qs], s_tree, -np.inf)
            mx = np.maximum(s_pre.max(axis=1, initial=-np.inf), s_tree.max(axis=1))
            e_pre = np.exp(s_pre - mx[:, None])
            e_tree = np.exp(s_tree - mx[:, None])                   # masked entries give exact zeros
            den = e_pre.sum(axis=1) + e_tree.sum(axis=1)
            num = e_pre @ pv[:, h] + e_tree @ vf[b, :, h]
            o[b, qs, h] = store(num / den[:, None])
    return o, k_rot


# ----------------------------------------------------------------------------
# 4. verifier logits and row statistics
# ----------------------------------------------------------------------------

def row_stats(z: np.ndarray, tau: float) -> Dict[str, float]:
    """max, argmax (smallest index among equal maxima), logZ and entropy of softmax(z/tau)."""
    amax = int(np.argmax(z))          # numpy returns the first maximal index
    mx = float(z[amax])
    if tau == 0.0:
        return {"max": mx, "argmax": amax, "logZ": 0.0, "H": 0.0}
    y = z / tau
    ym = y.max()
    e = np.exp(y - ym)
    S = e.sum()
    logZ = ym + math.log(S)
    p = e / S
    nz = p > 0
    H = float(-(p[nz] * np.log(p[nz])).sum())
    return {"max": mx, "argmax": amax, "logZ": float(logZ), "H": H}


def verify_logits(x: np.ndarray, Wlm, tau: float):
    """z'_r = W_lm x_r for every row r of x [R][d]; returns (logits [R][V], per-row stats)."""
    z = to_f64(x) @ to_f64(Wlm).T
    return z, [row_stats(z[r], tau) for r in range(z.shape[0])]


def edge_logits(z: np.ndarray, tokens: np.ndarray, tree: OracleTree):
    """edge[b][c] = z'_{b, parent(c)}[token c] for c >= 1 (edge[b][0] = 0)."""
    B, T = tokens.shape
    e = np.zeros((B, T))
    for b in range(B):
        for c in range(1, T):
            e[b, c] = z[b * T + tree.parent[c], tokens[b, c]]
    return e


# ----------------------------------------------------------------------------
# 5. acceptance
# ----------------------------------------------------------------------------

def edge_passes(mode: str, tok: int, par_stats, edge: float, eps: float, delta: float, tau: float) -> bool:
    """Does child token ``tok`` pass against the verifier distribution at its parent?"""
    if mode == "greedy":
        return tok == par_stats["argmax"]
    if mode != "typical":
        raise ValueError(mode)
    thr = min(eps, delta * math.exp(-par_stats["H"]))
    if tau == 0.0:
        p = 1.0 if tok == par_stats["argmax"] else 0.0
    else:
        p = math.exp(edge / tau - par_stats["logZ"])
    return p > thr


def accept_path(stats, edge, tokens, tree: OracleTree, mode: str, eps=0.09, delta=0.3, tau=0.0):
    """(paths: list of node-index lists root..leaf, n_acc list) for every sequence."""
    B, T = tokens.shape
    paths, n_acc = [], []
    for b in range(B):
        passed = [True] * T
        for c in range(1, T):
            p = tree.parent[c]
            passed[c] = edge_passes(mode, int(tokens[b, c]), stats[b * T + p], float(edge[b, c]), eps, delta, tau)
        best = 0
        for c in range(1, T):
            path = ancestors(tree, c)
            if all(passed[j] for j in path) and tree.depth[c] > tree.depth[best]:
                best = c
        path = ancestors(tree, best)
        paths.append(path)
        n_acc.append(len(path))
    return paths, n_acc


def softmax_tau(z: np.ndarray, tau: float) -> np.ndarray:
    """softmax(z / tau), max-shifted."""
    y = z / tau
    e = np.exp(y - y.max())
    return e / e.sum()


def inverse_cdf(r: np.ndarray, u: float) -> int:
    """Smallest index whose running sum of r exceeds u * sum(r) (u in [0, 1))."""
    c = np.cumsum(r)
    return int(min(np.searchsorted(c, u * c[-1], side="right"), r.shape[0] - 1))


def accept_rejection(z, head_logits, tokens, tree: OracleTree, tau: float, u_accept, u_resample, trace=None):
    """Rejection-sampling acceptance on the tree.

    Notes page ("Accelerating LLM Inference with Speculative Decoding: Notes on
    Medusa"), section 2, and the summary page's "Typical Acceptance Scheme" (first
    paragraph): a candidate x drafted with probability q(x) is accepted with
    probability min(1, p(x)/q(x)); on rejection the token is drawn from
    norm(max(0, p - q)).  On the tree: p is the verifier distribution softmax(z/tau)
    at the current node, q is the softmax(./tau) of the head whose candidates sit one
    level down.  Walking from the root, the children of the current node are tried in
    rank order, child c accepted iff u_accept[b][c] < min(1, r(x_c)/q(x_c)) with r the
    current residual (p at first); a rejection replaces r by norm(max(0, r - q)) before
    the next sibling.  An accepted child becomes the current node (r = its p).  When no
    child is accepted (or the node is a leaf) the next token is drawn from r by the
    inverse CDF at u_resample[b]; it is -1 when r has no mass left.

    Returns (paths root..last, n_acc, next_token) per sequence.  With ``trace`` (a list),
    every decision is appended as (b, u, threshold) for the acceptance tests and as
    (b, u * total, running sums) for the final draw, for margin checks.
    """
    B, T = tokens.shape
    kids = [[c for c in range(1, T) if tree.parent[c] == i] for i in range(T)]
    paths, n_acc, nxt = [], [], []
    for b in range(B):
        cur = 0
        path = [0]
        r = softmax_tau(z[b * T], tau)
        while True:
            d = tree.depth[cur]
            acc = None
            for c in kids[cur]:
                q = softmax_tau(head_logits[b, d + 1], tau)
                x = int(tokens[b, c])
                a = min(1.0, r[x] / q[x])
                if trace is not None:
                    trace.append(("accept", b, float(u_accept[b, c]), a))
                if u_accept[b, c] < a:
                    acc = c
                    break
                r = np.maximum(r - q, 0.0)
                tot = r.sum()
                if tot <= 0.0:
                    r = None
                    break
                r = r / tot
            if acc is None:
                break
            cur = acc
            path.append(cur)
            r = softmax_tau(z[b * T + cur], tau)
        paths.append(path)
        n_acc.append(len(path))
        nxt.append(-1 if r is None else inverse_cdf(r, float(u_resample[b])))
        if trace is not None and r is not None:
            trace.append(("draw", b, float(u_resample[b]), np.cumsum(r)))
    return paths, n_acc, nxt


# ----------------------------------------------------------------------------
# 6. KV compaction
# ----------------------------------------------------------------------------

def kv_compact(Kc, Vc, k_rot, v, paths, prefix_len, page_table=None, page_size=16):
    """Copies of the caches with the accepted rows appended at slots L_b .. L_b + n - 1."""
    Kn, Vn = Kc.copy(), Vc.copy()
    new_len = []
    for b, path in enumerate(paths):
        L = int(prefix_len[b])
        for j, node in enumerate(path):
            slot = L + j
            if page_table is None:
                Kn[b, slot] = k_rot[b, node]
                Vn[b, slot] = v[b, node]
            else:
                pg = page_table[b, slot // page_size]
                Kn[pg, slot % page_size] = k_rot[b, node]
                Vn[pg, slot % page_size] = v[b, node]
        new_len.append(L + len(path))
    return Kn, Vn, new_len


# ----------------------------------------------------------------------------
# whole step
# ----------------------------------------------------------------------------

def step(w, inp: dict, tree: OracleTree, mode: str, tau: float, eps=0.09, delta=0.3):
    """Run stages 1-6 on one set of inputs; returns a dict of every intermediate."""
    bf16 = w.dtype == "bf16"
    logits, a = medusa_heads(inp["h"], inp["W1"], inp["W2"], inp["Wlm"])
    B = w.B
    K1 = w.K + 1
    tk_idx = np.empty((B, K1, w.k_cfg), dtype=np.int64)
    tk_val = np.empty((B, K1, w.k_cfg))
    for b in range(B):
        for r in range(K1):
            tk_idx[b, r], tk_val[b, r] = topk(logits[b, r], w.k_cfg)
    tokens, pos = tree_expand(tk_idx, tree, inp["prefix_len"])
    pt = inp.get("page_table")
    o, k_rot = tree_attention(inp["q"], inp["k"], inp["v"], inp["Kc"], inp["Vc"], inp["prefix_len"], tree,
                              w.rope_theta, bf16_store=bf16, page_table=pt, page_size=w.page_size)
    x = o.reshape(B * tree.T, w.d)
    z, stats = verify_logits(x, inp["Wlm"], tau)
    edge = edge_logits(z, tokens, tree)
    paths, n_acc = accept_path(stats, edge, tokens, tree, mode, eps, delta, tau)
    vf = to_f64(inp["v"])
    Kn, Vn, new_len = kv_compact(to_f64(inp["Kc"]), to_f64(inp["Vc"]), k_rot, vf, paths, inp["prefix_len"],
                                 pt, w.page_size)
    return dict(logits=logits, a=a, topk_idx=tk_idx, topk_val=tk_val, tokens=tokens, pos=pos,
                o=o, k_rot=k_rot, x=x, z=z, stats=stats, edge=edge, paths=paths, n_acc=n_acc,
                K_new=Kn, V_new=Vn, new_len=new_len)


# ----------------------------------------------------------------------------
# chained steps (multi-step decoding)
# ----------------------------------------------------------------------------

def decode_loop(w, inp: dict, qkv_steps, tree: OracleTree, mode: str, tau: float, eps=0.09, delta=0.3):
    """Chain one step per entry of ``qkv_steps`` (the tree's q/k/v inputs of that step).

    Summary page, section 3.2: after acceptance the next iteration continues from
    the last accepted token.  Step s+1 starts from step s's result: its hidden state
    h is the node output of each sequence's deepest accepted node (whose LM-head
    row is that node's verifier row, so the next root is that row's argmax), its
    cache is the compacted one and its prefix length is the new length.  Weights
    stay the same.  Returns the list of step results.
    """
    state = {k: v for k, v in inp.items() if k not in ("q", "k", "v")}
    results = []
    for qkv in qkv_steps:
        cur = dict(state)
        cur.update(qkv)
        r = step(w, cur, tree, mode, tau, eps, delta)
        results.append(r)
        B = w.B
        state["h"] = np.stack([r["o"][b, r["paths"][b][-1]].reshape(w.d) for b in range(B)])
        state["Kc"], state["Vc"] = r["K_new"], r["V_new"]
        state["prefix_len"] = np.asarray(r["new_len"], dtype=np.int32)
    return results
