"""Oracle candidate trees: Cartesian and sparse (score-ranked), plus the tree mask.

A node is identified by its *rank path* ``(r_1, ..., r_l)``: the node at depth
``l`` carries the rank-``r_l`` candidate of Medusa head ``l`` and extends its
parent ``(r_1, ..., r_{l-1})``.  The root ``()`` is the LM head's top token.

Sources:
* Cartesian tree -- summary page, "Tree Attention" steps 1-2 (top-s_k per head,
  Cartesian product, level sizes are running products of the s_k); "Notes on
  Medusa" section 3 (node count sum_i prod_{j<=i} s_j).
* Sparse tree -- summary page, "Optimized Tree Construction" steps 2-4 (path
  accuracy is the product of per-head, per-rank accuracies under independence;
  nodes are added greedily from the frontier of the current tree); "Notes on
  Medusa" section 4 (expected acceptance length sums path products over all
  nodes).  The greedy step ranks candidates by their path product.  Ties are
  broken by smaller depth, then by the lexicographically smaller rank path.
* Mask -- summary page, "Tree Attention" step 3: node i may attend to node j
  iff j is an ancestor of i; the node itself is included (causal self-attention).
* Packing -- "Notes on Medusa" section 3 (the tree is flattened into one
  sequence): breadth-first, root first, then by depth, then by rank path.
"""

from __future__ import annotations

import heapq
import itertools
from dataclasses import dataclass
from fractions import Fraction
from typing import List, Sequence, Tuple

Path = Tuple[int, ...]


@dataclass
class OracleTree:
    paths: List[Path]          # BFS-packed; paths[0] == ()
    parent: List[int]          # parent[0] == -1
    depth: List[int]
    rank: List[int]            # last rank of the path (0 for the root)
    max_depth: int

    @property
    def T(self) -> int:
        return len(self.paths)


def _pack(paths: Sequence[Path]) -> OracleTree:
    order = sorted(set(paths), key=lambda p: (len(p), p))
    if not order or order[0] != ():
        raise ValueError("tree must contain the root")
    index = {p: i for i, p in enumerate(order)}
    parent, depth, rank = [], [], []
    for p in order:
        if p == ():
            parent.append(-1)
            rank.append(0)
        else:
            if p[:-1] not in index:
                raise ValueError(f"node {p} has no parent in the tree")
            parent.append(index[p[:-1]])
            rank.append(p[-1])
        depth.append(len(p))
    return OracleTree(list(order), parent, depth, rank, max(depth))


def cartesian_tree(s: Sequence[int]) -> OracleTree:
    """All rank paths (r_1..r_l), l <= K, with r_j < s_j: the Cartesian-product tree."""
    paths: List[Path] = [()]
    for level in range(1, len(s) + 1):
        paths.extend(itertools.product(*[range(s[j]) for j in range(level)]))
    return _pack(paths)


def path_score(path: Path, a0, rho, gamma, rank_base: int = 0, depth_base: int = 0) -> Fraction:
    """Exact product over the path of a0 * rho**(r_j + rank_base) * gamma**(j - 1 + depth_base)."""
    a0, rho, gamma = Fraction(str(a0)), Fraction(str(rho)), Fraction(str(gamma))
    s = Fraction(1)
    for j, r in enumerate(path, start=1):
        s *= a0 * rho ** (r + rank_base) * gamma ** (j - 1 + depth_base)
    return s


def _order_key(path: Path, score: Fraction):
    return (-score, len(path), path)


def scored_tree_greedy(K: int, k_cfg: int, T: int, a0=0.6, rho=0.7, gamma=0.8,
                       rank_base: int = 0, depth_base: int = 0) -> OracleTree:
    """Greedy frontier construction: repeatedly add the best frontier node until T nodes."""
    if T < 1:
        raise ValueError("T must count the root")
    sc = lambda p: path_score(p, a0, rho, gamma, rank_base, depth_base)
    chosen: List[Path] = [()]
    frontier = []  # heap of (order key, path)
    if K >= 1:
        for r in range(k_cfg):
            heapq.heappush(frontier, _order_key((r,), sc((r,))))
    while len(chosen) < T:
        if not frontier:
            raise ValueError("tree budget exceeds the number of candidate nodes")
        best = heapq.heappop(frontier)[2]
        chosen.append(best)
        if len(best) < K:
            for r in range(k_cfg):
                c = best + (r,)
                heapq.heappush(frontier, _order_key(c, sc(c)))
    return _pack(chosen)


def scored_tree_bruteforce(K: int, k_cfg: int, T: int, a0=0.6, rho=0.7, gamma=0.8,
                           rank_base: int = 0, depth_base: int = 0) -> OracleTree:
    """Enumerate every rank path up to depth K and keep the T-1 best (plus the root)."""
    allp = []
    for level in range(1, K + 1):
        allp.extend(itertools.product(range(k_cfg), repeat=level))
    scored = sorted(allp, key=lambda p: _order_key(p, path_score(p, a0, rho, gamma, rank_base, depth_base)))
    return _pack([()] + scored[:T - 1])


def expected_accept_length(tree: OracleTree, a0=0.6, rho=0.7, gamma=0.8,
                           rank_base: int = 0, depth_base: int = 0) -> Fraction:
    """Sum over all non-root nodes of the path product ("Notes on Medusa", section 4)."""
    return sum((path_score(p, a0, rho, gamma, rank_base, depth_base) for p in tree.paths[1:]), Fraction(0))


def table_product(path: Path, acc) -> float:
    """Product of acc[j][r_j] over the path, multiplied in path order in double precision.

    Summary page, "Optimized Tree Construction", step 2 (independence: a path's accuracy
    is the product of its nodes' accuracies).  The order between paths is decided in
    double precision, as the library does; expected lengths below are exact.
    """
    s = 1.0
    for j, r in enumerate(path):
        s *= float(acc[j][r])
    return s


def table_tree_greedy(K: int, k_cfg: int, T: int, acc) -> OracleTree:
    """Greedy frontier (steps 3-4; "Notes on Medusa", section 4) with table path products."""
    if T < 1:
        raise ValueError("T must count the root")
    chosen: List[Path] = [()]
    frontier = []
    for r in range(k_cfg):
        heapq.heappush(frontier, _order_key((r,), table_product((r,), acc)))
    while len(chosen) < T:
        if not frontier:
            raise ValueError("tree budget exceeds the number of candidate nodes")
        best = heapq.heappop(frontier)[2]
        chosen.append(best)
        if len(best) < K:
            for r in range(k_cfg):
                c = best + (r,)
                heapq.heappush(frontier, _order_key(c, table_product(c, acc)))
    return _pack(chosen)


def table_expected_length(tree: OracleTree, acc) -> Fraction:
    """E[L] = sum over the non-root nodes of the exact product of their accuracies."""
    tot = Fraction(0)
    for p in tree.paths[1:]:
        s = Fraction(1)
        for j, r in enumerate(p):
            s *= Fraction(float(acc[j][r]))
        tot += s
    return tot


def marginal_accuracy(top_i) -> List[float]:
    """Accuracy of the rank-i candidate from cumulative top-i accuracies: top-i minus top-(i-1)
    (summary page, "Optimized Tree Construction", step 1)."""
    out, prev = [], 0.0
    for c in top_i:
        out.append(float(c) - prev)
        prev = float(c)
    return out


def ancestor_mask(tree: OracleTree):
    """M[i][j] = True iff walking parent pointers from i reaches j (i itself included)."""
    T = tree.T
    M = [[False] * T for _ in range(T)]
    for i in range(T):
        j = i
        while j != -1:
            M[i][j] = True
            j = tree.parent[j]
    return M


def ancestors(tree: OracleTree, i: int) -> List[int]:
    """Root-to-i path of packed indices (root first, i last)."""
    out = []
    j = i
    while j != -1:
        out.append(j)
        j = tree.parent[j]
    return out[::-1]


def build_tree(w) -> OracleTree:
    """The tree a workload uses."""
    if w.tree_kind == "cartesian":
        return cartesian_tree(w.tree_s)
    return scored_tree_greedy(w.K, w.k_cfg, w.T, w.a0, w.rho, w.gamma)
