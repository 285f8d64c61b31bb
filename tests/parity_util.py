"""Shared helpers of the GPU parity tests: oracle runs, tolerance checks."""

from __future__ import annotations

import functools
import json
import os
import sys

import numpy as np

from oracle import margins as om
from oracle import step as ostep
from oracle import tree as otree
from workloads import make_inputs
from workloads.configs import get_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SEEDS = json.load(open(os.path.join(ROOT, "workloads", "seeds.json")))

# Floating-point bar: per row, max |gpu - oracle| / max |oracle| <= 2e-2.
REL_TOL = 2e-2


def note(*a):
    print("[parity]", *a, file=sys.stderr, flush=True)


def rel_err_rows(g: np.ndarray, r: np.ndarray) -> float:
    g = np.asarray(g, dtype=np.float64).reshape(-1, g.shape[-1])
    r = np.asarray(r, dtype=np.float64).reshape(-1, r.shape[-1])
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def bf16_f64(a: np.ndarray) -> np.ndarray:
    return ostep.to_f64(a)


def seed_of(name: str) -> int:
    return SEEDS[name]["seed"]


@functools.lru_cache(maxsize=None)
def case_inputs(name: str):
    w = get_case(name)
    return w, make_inputs(w, seed_of(name))


@functools.lru_cache(maxsize=None)
def oracle_shared(name: str):
    """Stages that do not depend on the acceptance run: heads, top-k, tree, attention, verifier logits."""
    w, inp = case_inputs(name)
    tree = otree.build_tree(w)
    logits, _ = ostep.medusa_heads(inp["h"], inp["W1"], inp["W2"], inp["Wlm"])
    K1 = w.K + 1
    tk_idx = np.empty((w.B, K1, w.k_cfg), dtype=np.int64)
    tk_val = np.empty((w.B, K1, w.k_cfg))
    for b in range(w.B):
        for r in range(K1):
            tk_idx[b, r], tk_val[b, r] = ostep.topk(logits[b, r], w.k_cfg)
    tokens, pos = ostep.tree_expand(tk_idx, tree, inp["prefix_len"])
    o, k_rot = ostep.tree_attention(inp["q"], inp["k"], inp["v"], inp["Kc"], inp["Vc"], inp["prefix_len"], tree,
                                    w.rope_theta, bf16_store=(w.dtype == "bf16"),
                                    page_table=inp.get("page_table"), page_size=w.page_size)
    x = o.reshape(w.B * tree.T, w.d)
    z = x @ ostep.to_f64(inp["Wlm"]).T
    return dict(tree=tree, logits=logits, topk_idx=tk_idx, topk_val=tk_val, tokens=tokens, pos=pos, o=o,
                k_rot=k_rot, x=x, z=z)


@functools.lru_cache(maxsize=None)
def oracle_run(name: str, run_idx: int):
    w, inp = case_inputs(name)
    sh = oracle_shared(name)
    run = w.accept[run_idx]
    stats = [ostep.row_stats(sh["z"][r], run.temperature) for r in range(sh["z"].shape[0])]
    edge = ostep.edge_logits(sh["z"], sh["tokens"], sh["tree"])
    paths, n_acc = ostep.accept_path(stats, edge, sh["tokens"], sh["tree"], run.mode, run.eps, run.delta,
                                     run.temperature)
    return dict(stats=stats, edge=edge, paths=paths, n_acc=n_acc, run=run)


def cache_row(C: np.ndarray, b: int, slot: int, page_table, page_size: int):
    if page_table is None:
        return C[b, slot]
    return C[page_table[b, slot // page_size], slot % page_size]


def unique_rows(z: np.ndarray):
    return set(om.unique_argmax_rows(z))


def exact_topk(row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values of a row, equal values by smaller index."""
    order = np.lexsort((np.arange(row.shape[0]), -np.asarray(row, dtype=np.float64)))
    return order[:k]


def clear_topk_rows(ref: np.ndarray, diff: np.ndarray, k: int) -> np.ndarray:
    """Per row of ``ref`` [..][V]: True where every gap between consecutive values of the
    top k+1 exceeds twice ``diff`` (that row's largest GPU-vs-oracle difference), so the
    top-k indices of two rows within ``diff`` of each other must agree."""
    top = -np.sort(-ref, axis=-1)[..., :k + 1]
    gaps = top[..., :-1] - top[..., 1:]
    return gaps.min(axis=-1) > 2 * diff

