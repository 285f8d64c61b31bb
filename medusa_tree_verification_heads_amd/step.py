"""One draft-and-verify step: the six library calls in order on one stream.

``VerifyStep`` uploads a workload's inputs once, allocates every output and
workspace once, and ``run()`` enqueues

    medusa_heads -> topk_tree_expand -> tree_attention -> verify_logits
    -> accept_path -> kv_compact

(the last two as the single launch accept_compact unless ``fused_tail=False``)
with no host synchronisation, so a step can also be captured in a HIP graph.
The order is the information flow of the summary page ("Medusa: Simple LLM
Inference Acceleration Framework with Multiple Decoding Heads", section 3.2).
"""

from __future__ import annotations

import numpy as np
import torch

from . import (GREEDY, TYPICAL, MDT_BF16, MDT_F32, KVCache, Tree, accept_compact, accept_path, kv_compact,
               medusa_heads,
               medusa_heads_workspace, new_workspace, topk_tree_expand, topk_workspace, tree_attention,
               tree_attention_workspace, verify_logits, verify_logits_workspace)


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """numpy array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class VerifyStep:
    def __init__(self, w, inp: dict, mode: str = "greedy", temperature: float = 0.0, eps: float = 0.09,
                 delta: float = 0.3, device="cuda", want_logits: bool = False, tree: Tree = None,
                 fused_tail: bool = True):
        self.w = w
        self.fused_tail = fused_tail
        self.mode = GREEDY if mode == "greedy" else TYPICAL
        self.temperature, self.eps, self.delta = float(temperature), float(eps), float(delta)
        dev = torch.device(device)
        self.dev = dev
        t = {k: to_device(inp[k], dev) for k in ("h", "W1", "W2", "Wlm", "Kc", "Vc", "q", "k", "v")}
        self.t = t
        self.prefix_len = torch.from_numpy(inp["prefix_len"].astype(np.int32)).to(dev)
        pt = inp.get("page_table")
        self.page_table = None if pt is None else torch.from_numpy(pt.astype(np.int32)).to(dev)
        self.cache = KVCache(t["Kc"], t["Vc"], self.page_table, w.page_size)
        self.tree = (tree or Tree.for_workload(w)).to_device(dev)
        B, d, V, K, k_cfg, T, H, Dh = w.B, w.d, w.V, w.K, w.k_cfg, self.tree.T, w.H, w.Dh
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.logits = torch.empty((B, K + 1, V), **f32)
        self.topk_idx = torch.empty((B, K + 1, k_cfg), **i32)
        self.topk_val = torch.empty((B, K + 1, k_cfg), **f32)
        self.tokens = torch.empty((B, T), **i32)
        self.pos = torch.empty((B, T), **i32)
        self.o = torch.empty_like(t["q"])
        self.k_rot = torch.empty_like(t["k"])
        self.stats = torch.empty((B * T, 4), **i32)
        self.edge = torch.empty((B, T), **f32)
        self.vlogits = torch.empty((B * T, V), **f32) if want_logits else None
        self.path = torch.empty((B, self.tree.tree.max_depth + 1), **i32)
        self.n_acc = torch.empty((B,), **i32)
        self.new_len = torch.empty((B,), **i32)
        dt = MDT_BF16 if w.dtype == "bf16" else MDT_F32
        self.ws_heads = new_workspace(medusa_heads_workspace(B, d, K), dev)
        self.ws_topk = new_workspace(topk_workspace(B, K, V, k_cfg), dev)
        self.ws_attn = new_workspace(tree_attention_workspace(dt, B, T, H, Dh, self.cache.desc.capacity), dev)
        self.ws_verify = new_workspace(verify_logits_workspace(dt, B, T, d, V), dev)

    def run(self, stream=None):
        t, w = self.t, self.w
        medusa_heads(t["h"], t["W1"], t["W2"], t["Wlm"], logits=self.logits, ws=self.ws_heads, stream=stream)
        topk_tree_expand(self.logits, w.k_cfg, self.tree, self.prefix_len, self.topk_idx, self.topk_val, self.tokens,
                         self.pos, ws=self.ws_topk, stream=stream)
        tree_attention(t["q"], t["k"], t["v"], self.cache, self.prefix_len, self.tree, w.rope_theta, out=self.o,
                       k_rot=self.k_rot, ws=self.ws_attn, stream=stream)
        x = self.o.view(w.B * self.tree.T, w.d)
        verify_logits(x, t["Wlm"], self.tree, self.tokens, self.temperature, stats=self.stats, edge=self.edge,
                      logits=self.vlogits, want_logits=self.vlogits is not None, ws=self.ws_verify, stream=stream)
        if self.fused_tail:
            accept_compact(self.stats, self.edge, self.tokens, self.tree, self.mode, self.eps, self.delta,
                           self.temperature, self.k_rot, t["v"], self.cache, self.prefix_len, path=self.path,
                           n_acc=self.n_acc, new_prefix_len=self.new_len, stream=stream)
            return
        accept_path(self.stats, self.edge, self.tokens, self.tree, self.mode, self.eps, self.delta, self.temperature,
                    path=self.path, n_acc=self.n_acc, stream=stream)
        kv_compact(self.path, self.n_acc, self.k_rot, t["v"], self.cache, self.prefix_len, self.new_len,
                   stream=stream)

    def outputs(self) -> dict:
        """Copies of every output on the host (synchronises)."""
        torch.cuda.synchronize()

        def f(x):
            if x is None:
                return None
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).cpu().numpy().view(np.uint16)
            return x.cpu().numpy()

        return dict(logits=f(self.logits), topk_idx=f(self.topk_idx), topk_val=f(self.topk_val),
                    tokens=f(self.tokens), pos=f(self.pos), o=f(self.o), k_rot=f(self.k_rot),
                    stats=f(self.stats).view(np.int32), edge=f(self.edge), vlogits=f(self.vlogits),
                    path=f(self.path), n_acc=f(self.n_acc), new_len=f(self.new_len),
                    Kc=f(self.t["Kc"]), Vc=f(self.t["Vc"]))
