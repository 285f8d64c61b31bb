"""Planted acceptance inputs: verifier row statistics, edge logits and tree tokens
chosen so that the accepted path lands at a chosen depth.

Random weights give verifier rows that are nearly flat, so a real step almost always
accepts either only the root (greedy) or the whole depth (typical).  These inputs
exercise the acceptance rule of the summary page ("Typical Acceptance Scheme": a
candidate is kept up to its first failing token, the longest accepted prefix over all
branches wins; "Notes on Medusa" section 3, the greedy walk) in between:

* every accepted length 1 .. max_depth + 1 (sequence b aims at depth b mod (D + 1));
* deep nodes whose own edge passes below an ancestor that fails (a rule that ignored
  ancestors would pick them);
* several accepted nodes at the deepest accepted depth (typical mode; the smallest
  packed index wins).

Only the pass/fail pattern is planted here; the expected result is always the
oracle's ``accept_path`` on the planted values.  Typical edges sit at least
``MARGIN`` (log-probability units) from their threshold, far above float32 rounding.
"""

from __future__ import annotations

import math

import numpy as np

MARGIN = 0.05
STATS_DTYPE = np.dtype([("max", np.float32), ("argmax", np.int32), ("logZ", np.float32), ("entropy", np.float32)])


def _anc_or_self(parent, c):
    out = []
    while c >= 0:
        out.append(c)
        c = parent[c]
    return out[::-1]


def planted_case(parent, depth, B, mode, tau, eps, delta, seed, V=4096, p_pass=0.6):
    """Planted inputs for B sequences over one tree (``parent``/``depth`` in packed order).

    Returns dict(tokens [B][T] int32, stats [B*T] STATS_DTYPE, edge [B][T] float32,
    stats_list (oracle dicts), target [B] (the node each sequence aims at)).
    """
    parent = [int(x) for x in parent]
    depth = [int(x) for x in depth]
    T = len(parent)
    D = max(depth)
    rng = np.random.default_rng(seed)
    children = [[] for _ in range(T)]
    for c in range(1, T):
        children[parent[c]].append(c)
    by_depth = [[i for i in range(T) if depth[i] == k] for k in range(D + 1)]
    greedy_like = mode == "greedy" or tau == 0.0

    tokens = np.zeros((B, T), dtype=np.int32)
    stats = np.zeros(B * T, dtype=STATS_DTYPE)
    edge = np.zeros((B, T), dtype=np.float32)
    targets = []
    for b in range(B):
        # siblings carry distinct tokens (distinct top-k entries of one head)
        tokens[b, 0] = rng.integers(0, V)
        for p in range(T):
            if children[p]:
                tokens[b, children[p]] = rng.choice(V, size=len(children[p]), replace=False)
        tgt_depth = b % (D + 1)
        t = int(rng.choice(by_depth[tgt_depth]))
        targets.append(t)
        on = set(_anc_or_self(parent, t))
        passes = rng.random(T) < p_pass
        passes[0] = True
        for j in on:
            passes[j] = True
        if greedy_like:
            # at most one child of a node can carry the verifier's top token
            for p in range(T):
                kids = [c for c in children[p] if passes[c]]
                if len(kids) > 1:
                    keep = [c for c in kids if c in on] or [int(rng.choice(kids))]
                    for c in kids:
                        passes[c] = c == keep[0]
        # nothing below the target depth may be reachable through passing edges
        acc = np.zeros(T, dtype=bool)
        acc[0] = True
        for c in range(1, T):
            if passes[c] and acc[parent[c]]:
                if depth[c] > tgt_depth:
                    passes[c] = False
                else:
                    acc[c] = True
        # realise the pattern as statistics and edge logits
        for p in range(T):
            r = b * T + p
            stats[r]["max"] = np.float32(rng.uniform(5, 15))
            if greedy_like:
                kid = [c for c in children[p] if passes[c]]
                if kid:
                    stats[r]["argmax"] = tokens[b, kid[0]]
                else:
                    taken = set(int(tokens[b, c]) for c in children[p])
                    a = int(rng.integers(0, V))
                    while a in taken:
                        a = (a + 1) % V
                    stats[r]["argmax"] = a
            else:
                stats[r]["argmax"] = int(rng.integers(0, V))
                stats[r]["logZ"] = np.float32(rng.uniform(1, 10))
                stats[r]["entropy"] = np.float32(rng.uniform(0.2, 5))
        if not greedy_like:
            for c in range(1, T):
                st = stats[b * T + parent[c]]
                thr = min(math.log(eps), math.log(delta) - float(st["entropy"]))
                m = rng.uniform(MARGIN * 2, 1.5)
                lp = thr + (m if passes[c] else -m)
                edge[b, c] = np.float32(tau * (lp + float(st["logZ"])))
    stats_list = [{"max": float(s["max"]), "argmax": int(s["argmax"]), "logZ": float(s["logZ"]),
                   "H": float(s["entropy"])} for s in stats]
    return dict(tokens=tokens, stats=stats, edge=edge, stats_list=stats_list, targets=targets)


def typical_margin(case, parent, tau, eps, delta) -> float:
    """Smallest |ln p - ln threshold| over all typical edges, from the stored float32 values."""
    B, T = case["tokens"].shape
    m = math.inf
    for b in range(B):
        for c in range(1, T):
            st = case["stats_list"][b * T + int(parent[c])]
            lp = float(case["edge"][b, c]) / tau - st["logZ"]
            thr = min(math.log(eps), math.log(delta) - st["H"])
            m = min(m, abs(lp - thr))
    return m


def coverage(case, n_acc, paths, parent, depth, mode, tau, eps, delta):
    """What a planted case exercises, from the oracle's result: the accepted lengths, the
    sequences with a passing edge below a failing ancestor deeper than the result, and the
    sequences with more than one accepted node at the deepest accepted depth."""
    B, T = case["tokens"].shape
    cut, ties = 0, 0
    for b in range(B):
        ok = [True] * T
        for c in range(1, T):
            st = case["stats_list"][b * T + int(parent[c])]
            if mode == "greedy" or tau == 0.0:
                ok[c] = int(case["tokens"][b, c]) == st["argmax"]
            else:
                lp = float(case["edge"][b, c]) / tau - st["logZ"]
                ok[c] = lp > min(math.log(eps), math.log(delta) - st["H"])
        accepted = [c for c in range(T) if all(ok[j] for j in _anc_or_self(parent, c))]
        deepest = n_acc[b] - 1
        if sum(1 for c in accepted if depth[c] == deepest) > 1:
            ties += 1
        if any(ok[c] and depth[c] > deepest and c not in accepted for c in range(1, T)):
            cut += 1
    return dict(lengths=sorted(set(n_acc)), cut=cut, ties=ties)
