"""Oracle of the full verify forward, in float64.  Test infrastructure only.

The summary page ("Medusa: Simple LLM Inference Acceleration Framework with
Multiple Decoding Heads", section 3.2 step 4, and "Tree Attention" steps 3-5) runs
the packed candidate tree through the whole backbone in one forward pass, with the
tree mask and depth positions in every attention layer, before the LM head gives
the verification logits; "Notes on Medusa", section 3, feeds the node outputs of
that pass to the LM head.  The pages name the backbone (Vicuna, a Llama model) but
do not spell out its layer, so the layer here is the Llama decoder layer:

    h = rmsnorm(x, g_attn);  q, k, v = h Wq^T, h Wk^T, h Wv^T
    o = tree attention of q, k, v over this layer's prefix cache (``step.tree_attention``)
    x = x + o Wo^T
    h = rmsnorm(x, g_mlp);   x = x + (silu(h Wg^T) * (h Wu^T)) Wd^T

with rmsnorm(x, g) = x / sqrt(mean(x^2) + eps) * g, no biases, weights stored
[out][in].  The first x is the embedding row of each node's token; after the last
layer a final rmsnorm gives the rows the LM head reads.  Each layer keeps its own
cache and, after acceptance, appends the accepted path's keys and values to it.

Storage points: the library stores in bf16 the normed rows, q/k/v, the attention
output, the residual stream after each addition, the SwiGLU product and the final
normed rows; the oracle rounds its float64 value to bf16 at exactly those points.
"""

from __future__ import annotations

import numpy as np

from . import step as ostep
from .tree import OracleTree


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Rows of x divided by their root mean square (plus eps under the root), times g; bf16."""
    ms = np.mean(x * x, axis=1, keepdims=True)
    return ostep.round_bf16(x / np.sqrt(ms + eps) * g[None, :])


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    return ostep.silu(gate) * up


def linear(x: np.ndarray, W: np.ndarray, residual=None) -> np.ndarray:
    """x W^T (W stored [out][in]) plus an optional residual, rounded to bf16 once."""
    y = x @ ostep.to_f64(W).T
    return ostep.round_bf16(y if residual is None else y + residual)


def decoder_layer(x, lw: dict, prefix_len, tree: OracleTree, w, eps: float):
    """One layer on the M = B*T tree rows x [M][d] (float64 holding bf16 values).

    Returns (x_out, k_rot, v): the new residual stream and the layer's rotated tree keys
    and values [B][T][H][Dh], which compaction appends to the layer's cache.
    """
    f = ostep.to_f64
    B, T = w.B, tree.T
    shp = (B, T, w.H, w.Dh)
    h = rmsnorm(x, f(lw["g_attn"]), eps)
    q, k, v = linear(h, lw["Wq"]), linear(h, lw["Wk"]), linear(h, lw["Wv"])
    o, k_rot = ostep.tree_attention(q.reshape(shp), k.reshape(shp), v.reshape(shp), lw["Kc"], lw["Vc"],
                                    prefix_len, tree, w.rope_theta, bf16_store=True)
    x = linear(o.reshape(B * T, w.d), lw["Wo"], x)
    h = rmsnorm(x, f(lw["g_mlp"]), eps)
    a = ostep.round_bf16(swiglu(h @ f(lw["Wg"]).T, h @ f(lw["Wu"]).T))
    x = linear(a, lw["Wd"], x)
    return x, k_rot, v.reshape(shp)


def forward(dw, inp: dict, fin: dict, layers, tree: OracleTree, mode: str, tau: float, eps=0.09, delta=0.3):
    """The step with the full forward in place of given q/k/v: heads, top-k, tree, then
    embedding -> layers -> final norm -> verifier logits -> acceptance -> per-layer
    compaction.  ``layers`` is a list of per-layer dicts (weights, Kc, Vc)."""
    w = dw.base
    B, T = w.B, tree.T
    logits, _ = ostep.medusa_heads(inp["h"], inp["W1"], inp["W2"], inp["Wlm"])
    K1 = w.K + 1
    tk_idx = np.empty((B, K1, w.k_cfg), dtype=np.int64)
    for b in range(B):
        for r in range(K1):
            tk_idx[b, r], _ = ostep.topk(logits[b, r], w.k_cfg)
    tokens, pos = ostep.tree_expand(tk_idx, tree, inp["prefix_len"])
    x = ostep.to_f64(fin["E"])[tokens.reshape(-1)]
    k_rots, vs = [], []
    for lw in layers:
        x, k_rot, v = decoder_layer(x, lw, inp["prefix_len"], tree, w, dw.norm_eps)
        k_rots.append(k_rot)
        vs.append(v)
    xf = rmsnorm(x, ostep.to_f64(fin["g_final"]), dw.norm_eps)
    z, stats = ostep.verify_logits(xf, inp["Wlm"], tau)
    edge = ostep.edge_logits(z, tokens, tree)
    paths, n_acc = ostep.accept_path(stats, edge, tokens, tree, mode, eps, delta, tau)
    caches = []
    new_len = [int(inp["prefix_len"][b]) + len(paths[b]) for b in range(B)]
    for lw, k_rot, v in zip(layers, k_rots, vs):
        Kn, Vn, _ = ostep.kv_compact(ostep.to_f64(lw["Kc"]), ostep.to_f64(lw["Vc"]), k_rot, v, paths,
                                     inp["prefix_len"])
        caches.append((Kn, Vn))
    return dict(logits=logits, topk_idx=tk_idx, tokens=tokens, pos=pos, x_last=x, xf=xf, z=z, stats=stats,
                edge=edge, paths=paths, n_acc=n_acc, k_rot=k_rots, v=vs, caches=caches, new_len=new_len)


def forward_loop(dw, inp: dict, fin: dict, layers, tree: OracleTree, steps: int, mode: str, tau: float, eps=0.09,
                 delta=0.3):
    """Chain ``steps`` forward steps (summary page, section 3.2: the next iteration
    continues from the last accepted token).  Step s+1's hidden state is the final normed
    row (the LM head's input) of each sequence's deepest accepted node, its prefix length
    the new length, and every layer's cache the compacted one.  Returns the step results."""
    w = dw.base
    cur = dict(inp)
    lays = [dict(lw) for lw in layers]
    out = []
    for _ in range(steps):
        r = forward(dw, cur, fin, lays, tree, mode, tau, eps, delta)
        out.append(r)
        T = tree.T
        cur = dict(cur)
        cur["h"] = np.stack([r["xf"][b * T + r["paths"][b][-1]] for b in range(w.B)])
        cur["prefix_len"] = np.asarray(r["new_len"], dtype=np.int32)
        for lw, (Kn, Vn) in zip(lays, r["caches"]):
            lw["Kc"], lw["Vc"] = Kn, Vn
    return out

