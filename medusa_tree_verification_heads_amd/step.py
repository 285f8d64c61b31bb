"""One draft-and-verify step: the six library calls in order on one stream.

``VerifyStep`` uploads a workload's inputs once, allocates every output and
workspace once, and ``run()`` enqueues

    medusa_heads -> topk_tree_expand -> tree_attention -> verify_logits
    -> accept_path -> kv_compact

(by default the last two as the single launch accept_compact; ``tail`` can select
verify_accept_compact -- the verifier's tiles, then one launch per sequence that merges
the row statistics, accepts and compacts -- and ``fused_tail=False`` the separate calls)
with no host synchronisation, so a step can also be captured in a HIP graph.
The order is the information flow of the summary page ("Medusa: Simple LLM
Inference Acceleration Framework with Multiple Decoding Heads", section 3.2).
With mode "rejection" the acceptance is accept_rejection followed by kv_compact.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (GREEDY, TYPICAL, MDT_BF16, MDT_F32, KVCache, Tree, accept_compact, accept_path, verify_accept_compact,
               accept_rejection, kv_compact, medusa_heads, next_logits, next_state,
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
                 fused_tail: bool = True, tail: str = "accept_compact"):
        self.w = w
        if mode not in ("greedy", "typical", "rejection"):
            raise ValueError(f"unknown acceptance mode {mode!r} (greedy, typical or rejection)")
        # rejection sampling (mode "rejection") reads full verifier rows and the step's
        # uniforms (inp["u_accept"], inp["u_resample"]); its acceptance and compaction are
        # two calls
        self.rejection = mode == "rejection"
        want_logits = want_logits or self.rejection
        # how the step ends: "verify_accept_compact" (verifier tiles, then merge, acceptance and
        # compaction in one launch), "accept_compact" (verify_logits, then acceptance and
        # compaction in one launch) or "separate" (the three calls); all write the same bits
        if tail not in ("verify_accept_compact", "accept_compact", "separate"):
            raise ValueError(f"unknown tail {tail!r}")
        self.tail = "separate" if (not fused_tail or self.rejection) else tail
        self.fused_tail = self.tail != "separate"
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
        self.next_token = torch.full((B,), -1, **i32)
        if self.rejection:
            self.u_accept = torch.from_numpy(np.ascontiguousarray(inp["u_accept"], dtype=np.float32)).to(dev)
            self.u_resample = torch.from_numpy(np.ascontiguousarray(inp["u_resample"], dtype=np.float32)).to(dev)
        dt = MDT_BF16 if w.dtype == "bf16" else MDT_F32
        self.ws_heads = new_workspace(medusa_heads_workspace(B, d, K), dev)
        self.ws_topk = new_workspace(topk_workspace(B, K, V, k_cfg), dev)
        self.ws_attn = new_workspace(tree_attention_workspace(dt, B, T, H, Dh, self.cache.desc.capacity), dev)
        self.ws_verify = new_workspace(verify_logits_workspace(dt, B, T, d, V), dev)

    def run(self, stream=None, h=None, qkv=None, prefix_len=None, new_prefix_len=None, tokens=None, path=None,
            n_acc=None, vlogits=None, lm_head=True):
        """Enqueue one step.  The keyword arguments replace the step's own input or output
        tensors for this call (a chain of steps passes each step's own); ``vlogits`` is a
        buffer for the verifier's full logits, and ``lm_head=False`` leaves the heads'
        slot 0 as it is (already filled by ``next_logits``)."""
        t, w = self.t, self.w
        h = t["h"] if h is None else h
        q, k, v = (t["q"], t["k"], t["v"]) if qkv is None else qkv
        prefix_len = self.prefix_len if prefix_len is None else prefix_len
        new_len = self.new_len if new_prefix_len is None else new_prefix_len
        tokens = self.tokens if tokens is None else tokens
        path = self.path if path is None else path
        n_acc = self.n_acc if n_acc is None else n_acc
        vlogits = self.vlogits if vlogits is None else vlogits
        medusa_heads(h, t["W1"], t["W2"], t["Wlm"] if lm_head else None, logits=self.logits, ws=self.ws_heads,
                     stream=stream)
        topk_tree_expand(self.logits, w.k_cfg, self.tree, prefix_len, self.topk_idx, self.topk_val, tokens,
                         self.pos, ws=self.ws_topk, stream=stream)
        tree_attention(q, k, v, self.cache, prefix_len, self.tree, w.rope_theta, out=self.o,
                       k_rot=self.k_rot, ws=self.ws_attn, stream=stream)
        x = self.o.view(w.B * self.tree.T, w.d)
        if self.tail == "verify_accept_compact":
            verify_accept_compact(x, t["Wlm"], self.tree, tokens, self.temperature, self.mode, self.eps, self.delta,
                                  self.k_rot, v, self.cache, prefix_len, stats=self.stats, edge=self.edge,
                                  logits=vlogits, want_logits=vlogits is not None, path=path, n_acc=n_acc,
                                  new_prefix_len=new_len, ws=self.ws_verify, stream=stream)
            return
        verify_logits(x, t["Wlm"], self.tree, tokens, self.temperature, stats=self.stats, edge=self.edge,
                      logits=vlogits, want_logits=vlogits is not None, ws=self.ws_verify, stream=stream)
        if self.rejection:
            accept_rejection(vlogits, self.logits, tokens, self.tree, self.temperature, self.u_accept,
                             self.u_resample, path=path, n_acc=n_acc, next_token=self.next_token, stream=stream)
            kv_compact(path, n_acc, self.k_rot, v, self.cache, prefix_len, new_len, stream=stream)
            return
        if self.tail == "accept_compact":
            accept_compact(self.stats, self.edge, tokens, self.tree, self.mode, self.eps, self.delta,
                           self.temperature, self.k_rot, v, self.cache, prefix_len, path=path,
                           n_acc=n_acc, new_prefix_len=new_len, stream=stream)
            return
        accept_path(self.stats, self.edge, tokens, self.tree, self.mode, self.eps, self.delta, self.temperature,
                    path=path, n_acc=n_acc, stream=stream)
        kv_compact(path, n_acc, self.k_rot, v, self.cache, prefix_len, new_len, stream=stream)

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
                    path=f(self.path), n_acc=f(self.n_acc), new_len=f(self.new_len), next_token=f(self.next_token),
                    Kc=f(self.t["Kc"]), Vc=f(self.t["Vc"]))


class DecodeLoop:
    """Chained steps on one stream (multi-step decoding).

    Step s+1 starts from step s: its hidden state is the node output of each
    sequence's deepest accepted node (``next_state``), its prefix length is step s's
    new length, and the cache already holds step s's accepted keys and values.  The
    tree's q/k/v inputs of every step are given (``qkv_steps``).  Every step reads
    and writes its own prefix-length, hidden-state, token, path and n_acc tensors,
    so ``run()`` can be repeated (or replayed as a graph) from the same start.

    With ``reuse_lm_head`` (the default) the verifier also writes its full logits, and
    step s+1's LM-head slot is step s's verifier row of the same node (``next_logits``,
    enqueued at the start of step s+1, so that step s's own slot stays readable until
    then): that row is W_lm applied to the next hidden state, so the heads skip their
    W_lm stream on every step after the first.
    """

    def __init__(self, w, inp: dict, qkv_steps, mode: str = "greedy", temperature: float = 0.0, eps: float = 0.09,
                 delta: float = 0.3, device="cuda", fused_tail: bool = True, want_logits: bool = False,
                 step: VerifyStep = None, reuse_lm_head: bool = True):
        # the chain takes each next root from the LM-head row, so a sampled next token (the
        # rejection sampler's) has nowhere to go: chaining it is not supported
        if (step.rejection if step is not None else mode == "rejection"):
            raise ValueError("DecodeLoop does not chain rejection sampling")
        # an existing step (same inputs) can be reused: the chain only adds its own state tensors
        self.step = step or VerifyStep(w, inp, mode, temperature, eps, delta, device, want_logits=want_logits,
                                       fused_tail=fused_tail)
        st = self.step
        self.S = len(qkv_steps)
        dev = st.dev
        self.qkv = [tuple(to_device(q[n], dev) for n in ("q", "k", "v")) for q in qkv_steps]
        S, B, T = self.S, w.B, st.tree.T
        self.h = [st.t["h"]] + [torch.empty_like(st.t["h"]) for _ in range(S)]
        self.lens = [st.prefix_len] + [torch.empty_like(st.prefix_len) for _ in range(S)]
        i32 = dict(dtype=torch.int32, device=dev)
        self.tokens = torch.empty((S, B, T), **i32)
        self.paths = torch.empty((S, B, st.path.shape[1]), **i32)
        self.n_acc = torch.empty((S, B), **i32)
        self.reuse = reuse_lm_head
        self.vlogits = st.vlogits
        if self.reuse and self.vlogits is None:
            self.vlogits = torch.empty((B * T, w.V), dtype=torch.float32, device=dev)

    def run_step(self, s: int, stream=None):
        st, w = self.step, self.step.w
        reuse = self.reuse and s > 0
        if reuse:
            next_logits(self.vlogits, self.paths[s - 1], self.n_acc[s - 1], st.logits, stream=stream)
        st.run(stream, h=self.h[s], qkv=self.qkv[s], prefix_len=self.lens[s], new_prefix_len=self.lens[s + 1],
               tokens=self.tokens[s], path=self.paths[s], n_acc=self.n_acc[s], vlogits=self.vlogits,
               lm_head=not reuse)
        next_state(st.o.view(w.B, st.tree.T, w.d), self.paths[s], self.n_acc[s], out=self.h[s + 1], stream=stream)

    def run(self, stream=None):
        for s in range(self.S):
            self.run_step(s, stream)
