"""The step with the full verify forward: the tree goes through every decoder layer.

The summary page ("Medusa: Simple LLM Inference Acceleration Framework with
Multiple Decoding Heads", section 3.2 step 4 and "Tree Attention" steps 3-5) runs
all candidates through the backbone in one forward pass with the tree mask before
the LM head.  ``VerifyForward.run()`` enqueues, on one stream and with no host
synchronisation:

    medusa_heads -> topk_tree_expand -> embed
    -> rmsnorm -> per layer: linear (q|k|v) -> tree_attention
                             -> linear_split (o Wo^T, slices) -> add_rmsnorm (x += ., h = norm)
                             -> linear (SwiGLU) -> linear_split (a Wd^T)
                             -> add_rmsnorm (x += ., h = next layer's norm, or the final one)
    -> verify_logits -> accept_path -> kv_compact_layers

The output and down projections have only d output columns (64 tiles of 64 at 7B), so
their inner dimension is cut into slices (linear_split; 4 at 7B, one 8-wave workgroup
per CU) whose fp32 products the following add_rmsnorm sums into the residual stream;
with one slice they are a plain linear with the residual in its epilogue followed by
rmsnorm.

Every layer has its own prefix cache (one allocation [layers][B][capacity][H][Dh]);
every layer's tree keys/values are kept until acceptance, then the accepted path is
appended to every layer's cache in one launch.
"""

from __future__ import annotations

from typing import List

import numpy as np
import torch

from . import (ACT_SWIGLU, GREEDY, TYPICAL, KVCache, Tree, accept_path, add_rmsnorm, auto_split, embed,
               interleave_gate_up, kv_compact_layers, linear, linear_split, medusa_heads, medusa_heads_workspace,
               new_workspace, next_logits, next_state, rmsnorm, topk_tree_expand, topk_workspace, tree_attention,
               tree_attention_workspace, verify_logits, verify_logits_workspace, MDT_BF16)
from .step import to_device

LAYER_KEYS = ("g_attn", "Wqkv", "Wo", "g_mlp", "Wgu", "Wd")


def upload_layer(lw: dict, device) -> dict:
    """One layer's numpy weights (bf16 patterns) -> the device layout the calls take:
    q|k|v stacked into one [3d][d] weight, gate/up interleaved by 16 rows."""
    t = {k: to_device(lw[k], device) for k in ("g_attn", "Wq", "Wk", "Wv", "Wo", "g_mlp", "Wg", "Wu", "Wd")}
    return {"g_attn": t["g_attn"], "Wqkv": torch.cat((t["Wq"], t["Wk"], t["Wv"])).contiguous(), "Wo": t["Wo"],
            "g_mlp": t["g_mlp"], "Wgu": interleave_gate_up(t["Wg"], t["Wu"]), "Wd": t["Wd"]}


class VerifyForward:
    """``base``: device tensors h, W1, W2, Wlm (the step's); ``E``, ``g_final``: embedding and
    final norm gain; ``layers``: per-layer dicts with LAYER_KEYS; ``Kc``/``Vc``: the caches
    of every layer, [n_layers][B][capacity][H][Dh]; ``prefix_len``: device int32 [B]."""

    def __init__(self, dw, base: dict, E, g_final, layers: List[dict], Kc, Vc, prefix_len, mode="greedy",
                 temperature=0.0, eps=0.09, delta=0.3, tree: Tree = None, splits=None):
        w = dw.base
        assert w.dtype == "bf16" and not w.paged, "the full forward runs on bf16 contiguous caches"
        self.dw, self.w = dw, w
        if mode not in ("greedy", "typical"):
            raise ValueError(f"unknown acceptance mode {mode!r} (greedy or typical)")
        self.mode = GREEDY if mode == "greedy" else TYPICAL
        self.temperature, self.eps, self.delta = float(temperature), float(eps), float(delta)
        self.base, self.E, self.g_final, self.layers = base, E, g_final, layers
        self.Kc, self.Vc, self.prefix_len = Kc, Vc, prefix_len
        dev = E.device
        self.dev = dev
        nL = len(layers)
        self.caches = [KVCache(Kc[l], Vc[l]) for l in range(nL)]
        self.tree = (tree or Tree.for_workload(w)).to_device(dev)
        B, d, V, K, k_cfg, T, H, Dh, F = w.B, w.d, w.V, w.K, w.k_cfg, self.tree.T, w.H, w.Dh, dw.ffn
        M = B * T
        self.M = M
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.logits = torch.empty((B, K + 1, V), **f32)
        self.topk_idx = torch.empty((B, K + 1, k_cfg), **i32)
        self.topk_val = torch.empty((B, K + 1, k_cfg), **f32)
        self.tokens = torch.empty((B, T), **i32)
        self.pos = torch.empty((B, T), **i32)
        self.x = torch.empty((M, d), **bf)
        self.h = torch.empty((M, d), **bf)
        self.qkv = torch.empty((nL, 3, M, d), **bf)      # per layer: q, k, v segments
        self.o = torch.empty((M, d), **bf)
        self.k_rot = torch.empty((nL, B, T, H, Dh), **bf)
        self.a = torch.empty((M, F), **bf)
        self.xf = torch.empty((M, d), **bf)
        self.stats = torch.empty((M, 4), **i32)
        self.edge = torch.empty((B, T), **f32)
        self.path = torch.empty((B, self.tree.tree.max_depth + 1), **i32)
        self.n_acc = torch.empty((B,), **i32)
        self.new_len = torch.empty((B,), **i32)
        self.ws_heads = new_workspace(medusa_heads_workspace(B, d, K), dev)
        self.ws_topk = new_workspace(topk_workspace(B, K, V, k_cfg), dev)
        self.ws_attn = new_workspace(tree_attention_workspace(MDT_BF16, B, T, H, Dh, self.caches[0].desc.capacity),
                                     dev) if nL else None
        self.ws_verify = new_workspace(verify_logits_workspace(MDT_BF16, B, T, d, V), dev)
        # slices of the output (o Wo^T) and down (a Wd^T) projections
        self.split_o, self.split_d = splits or (auto_split(M, d, d, dev), auto_split(M, d, F, dev))
        self.part = torch.empty((max(self.split_o, self.split_d), M, d), **f32)

    @classmethod
    def from_numpy(cls, dw, inp: dict, fin: dict, layers_np: List[dict], device="cuda", **kw):
        dev = torch.device(device)
        base = {k: to_device(inp[k], dev) for k in ("h", "W1", "W2", "Wlm")}
        layers = [upload_layer(lw, dev) for lw in layers_np]
        Kc = torch.stack([to_device(lw["Kc"], dev) for lw in layers_np]) if layers_np else None
        Vc = torch.stack([to_device(lw["Vc"], dev) for lw in layers_np]) if layers_np else None
        lens = torch.from_numpy(inp["prefix_len"].astype(np.int32)).to(dev)
        return cls(dw, base, to_device(fin["E"], dev), to_device(fin["g_final"], dev), layers, Kc, Vc, lens, **kw)

    def _close(self, a, W, nsplit, g, out, stream):
        """x += a W^T, then out = rmsnorm(x) * g."""
        eps = self.dw.norm_eps
        if nsplit > 1:
            part = self.part[:nsplit]
            linear_split(a, W, nsplit, out=part, stream=stream)
            add_rmsnorm(part, self.x, g, eps, out=out, stream=stream)
        else:
            linear(a, W, residual=self.x, out=self.x, stream=stream)
            rmsnorm(self.x, g, eps, out=out, stream=stream)

    def layer(self, l: int, stream=None, prefix_len=None):
        """Enqueue decoder layer l: self.h holds rmsnorm(x) * g_attn of this layer on entry;
        on exit self.x is the new residual stream and self.h (or, after the last layer,
        self.xf) its norm for what follows."""
        w, lw = self.w, self.layers[l]
        prefix_len = self.prefix_len if prefix_len is None else prefix_len
        B, T, H, Dh = w.B, self.tree.T, w.H, w.Dh
        qkv = self.qkv[l]
        linear(self.h, lw["Wqkv"], nseg=3, out=qkv, stream=stream)
        shp = (B, T, H, Dh)
        tree_attention(qkv[0].view(shp), qkv[1].view(shp), qkv[2].view(shp), self.caches[l], prefix_len,
                       self.tree, w.rope_theta, out=self.o.view(shp), k_rot=self.k_rot[l], ws=self.ws_attn,
                       stream=stream)
        self._close(self.o, lw["Wo"], self.split_o, lw["g_mlp"], self.h, stream)
        linear(self.h, lw["Wgu"], act=ACT_SWIGLU, out=self.a, stream=stream)
        last = l + 1 == len(self.layers)
        self._close(self.a, lw["Wd"], self.split_d, self.g_final if last else self.layers[l + 1]["g_attn"],
                    self.xf if last else self.h, stream)

    def run(self, stream=None, h=None, prefix_len=None, new_prefix_len=None, tokens=None, path=None,
            n_acc=None, vlogits=None, lm_head=True):
        """Enqueue one step.  The keyword arguments replace the step's own input or output
        tensors for this call (a chain of steps passes each step's own); ``vlogits`` receives
        the verifier's full logits, and ``lm_head=False`` leaves the heads' slot 0 as it is
        (already filled by ``next_logits``)."""
        w, t = self.w, self.base
        h = t["h"] if h is None else h
        prefix_len = self.prefix_len if prefix_len is None else prefix_len
        new_len = self.new_len if new_prefix_len is None else new_prefix_len
        tokens = self.tokens if tokens is None else tokens
        path = self.path if path is None else path
        n_acc = self.n_acc if n_acc is None else n_acc
        medusa_heads(h, t["W1"], t["W2"], t["Wlm"] if lm_head else None, logits=self.logits, ws=self.ws_heads,
                     stream=stream)
        topk_tree_expand(self.logits, w.k_cfg, self.tree, prefix_len, self.topk_idx, self.topk_val,
                         tokens, self.pos, ws=self.ws_topk, stream=stream)
        embed(tokens.view(-1), self.E, out=self.x, stream=stream)
        g0 = self.layers[0]["g_attn"] if self.layers else self.g_final
        rmsnorm(self.x, g0, self.dw.norm_eps, out=self.h if self.layers else self.xf, stream=stream)
        for l in range(len(self.layers)):
            self.layer(l, stream, prefix_len)
        verify_logits(self.xf, t["Wlm"], self.tree, tokens, self.temperature, stats=self.stats,
                      edge=self.edge, logits=vlogits, want_logits=vlogits is not None, ws=self.ws_verify,
                      stream=stream)
        accept_path(self.stats, self.edge, tokens, self.tree, self.mode, self.eps, self.delta,
                    self.temperature, path=path, n_acc=n_acc, stream=stream)
        if self.layers:
            B, T, H, Dh = w.B, self.tree.T, w.H, w.Dh
            v = self.qkv[:, 2].view(len(self.layers), B, T, H, Dh)
            kv_compact_layers(path, n_acc, self.k_rot, v, self.caches[0], prefix_len,
                              self.Kc.stride(0), new_prefix_len=new_len, stream=stream)

    def outputs(self) -> dict:
        torch.cuda.synchronize()

        def f(x):
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).cpu().numpy().view(np.uint16)
            return x.cpu().numpy()

        out = dict(logits=f(self.logits), tokens=f(self.tokens), x_last=f(self.x), xf=f(self.xf),
                   stats=f(self.stats).view(np.int32), edge=f(self.edge), path=f(self.path), n_acc=f(self.n_acc),
                   k_rot=f(self.k_rot), v=f(self.qkv[:, 2]))
        if self.layers:
            out.update(new_len=f(self.new_len), Kc=f(self.Kc), Vc=f(self.Vc))
        return out


class ForwardLoop:
    """Chained steps of the full forward (multi-step decoding through every layer).

    Step s+1 starts from step s: its hidden state is the final normed row (what the LM
    head reads) of each sequence's deepest accepted node (``next_state``), its prefix
    length is step s's new length, and every layer's cache already holds step s's
    accepted keys and values.  Every step has its own hidden-state, prefix-length, token,
    path and n_acc tensors, so ``run()`` can be repeated (or replayed as a graph) from the
    same start; the caches need room for one accepted path per step.  As in the single-layer
    chain, step s+1's LM-head slot is step s's verifier row of the same node
    (``next_logits``, unless ``reuse_lm_head=False``), so the heads skip W_lm after step 0.
    """

    def __init__(self, fwd: VerifyForward, steps: int, reuse_lm_head: bool = True):
        self.f = fwd
        self.S = steps
        self.reuse = reuse_lm_head
        self.vlogits = (torch.empty((fwd.w.B * fwd.tree.T, fwd.w.V), dtype=torch.float32, device=fwd.dev)
                        if reuse_lm_head else None)
        B, T = fwd.w.B, fwd.tree.T
        dev = fwd.dev
        h0 = fwd.base["h"]
        self.h = [h0] + [torch.empty_like(h0) for _ in range(steps)]
        self.lens = [fwd.prefix_len] + [torch.empty_like(fwd.prefix_len) for _ in range(steps)]
        i32 = dict(dtype=torch.int32, device=dev)
        self.tokens = torch.empty((steps, B, T), **i32)
        self.paths = torch.empty((steps, B, fwd.path.shape[1]), **i32)
        self.n_acc = torch.empty((steps, B), **i32)

    def run_step(self, s: int, stream=None):
        f = self.f
        reuse = self.reuse and s > 0
        if reuse:
            next_logits(self.vlogits, self.paths[s - 1], self.n_acc[s - 1], f.logits, stream=stream)
        f.run(stream, h=self.h[s], prefix_len=self.lens[s], new_prefix_len=self.lens[s + 1], tokens=self.tokens[s],
              path=self.paths[s], n_acc=self.n_acc[s], vlogits=self.vlogits, lm_head=not reuse)
        next_state(f.xf.view(f.w.B, f.tree.T, f.w.d), self.paths[s], self.n_acc[s], out=self.h[s + 1], stream=stream)

    def run(self, stream=None):
        for s in range(self.S):
            self.run_step(s, stream)

