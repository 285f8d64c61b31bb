"""Pins of the oracle's candidate trees and tree mask (CPU only)."""

import itertools
import json
import os
from fractions import Fraction

import pytest

from oracle import tree as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_cartesian_counts_printed_on_pages():
    g = json.load(open(os.path.join(GOLDEN, "cartesian_counts.json")))
    for case in g["cases"]:
        t = ot.cartesian_tree(case["s"])
        assert t.T - 1 == case["tokens"]
        leaves = [i for i in range(t.T) if t.depth[i] == len(case["s"])]
        assert len(leaves) == case["paths"]


def test_cartesian_level_sizes_are_running_products():
    # summary page, "Tree Attention" step 2: level k holds prod_{i<=k} s_i nodes
    s = (3, 2, 4)
    t = ot.cartesian_tree(s)
    prod = 1
    for lvl, sk in enumerate(s, start=1):
        prod *= sk
        assert sum(1 for dd in t.depth if dd == lvl) == prod


def _check_invariants(t):
    assert t.paths[0] == () and t.parent[0] == -1 and t.depth[0] == 0
    for i in range(1, t.T):
        p = t.parent[i]
        assert 0 <= p < i
        assert t.depth[i] == t.depth[p] + 1
        assert t.paths[p] == t.paths[i][:-1]
        assert t.rank[i] == t.paths[i][-1]
    # breadth-first packing: depth non-decreasing, rank paths ascending within a depth
    keys = [(len(p), p) for p in t.paths]
    assert keys == sorted(keys)


@pytest.mark.parametrize("K,k,T", [(2, 3, 8), (3, 6, 40), (4, 10, 42), (4, 10, 64), (5, 4, 100), (3, 5, 124)])
def test_sparse_greedy_equals_bruteforce(K, k, T):
    g = ot.scored_tree_greedy(K, k, T)
    b = ot.scored_tree_bruteforce(K, k, T)
    assert g.paths == b.paths
    _check_invariants(g)


def test_sparse_tree_alternative_depth_base():
    g = ot.scored_tree_greedy(4, 10, 64, depth_base=1, rank_base=0)
    b = ot.scored_tree_bruteforce(4, 10, 64, depth_base=1, rank_base=0)
    assert g.paths == b.paths


def test_sparse_tree_64_nodes_depth4_leans_left():
    # summary page, "Optimized Tree Construction": the 64-node tree of Figure 6 has depth 4 and
    # leans to the left (higher-ranked candidates get more descendants).
    t = ot.scored_tree_greedy(4, 10, 64)
    assert t.T == 64 and t.max_depth == 4
    present = set(t.paths)
    for p in t.paths[1:]:
        if p[-1] > 0:
            assert p[:-1] + (p[-1] - 1,) in present      # left sibling present
        # a lower-ranked ancestor choice never has more depth below it than the higher-ranked one
    sub = {}
    for p in t.paths[1:]:
        sub[p[0]] = sub.get(p[0], 0) + 1
    counts = [sub.get(r, 0) for r in range(10)]
    assert counts == sorted(counts, reverse=True)


def test_sparse_tree_exact_tie_handling():
    # scores a0^l * rho^R * gamma^D with a0=3/5, rho=7/10, gamma=4/5 tie exactly iff (l, R, D) tie
    p1, p2 = (0, 1), (1, 0)            # l=2, R=1, D=1 for both
    s1 = ot.path_score(p1, 0.6, 0.7, 0.8)
    s2 = ot.path_score(p2, 0.6, 0.7, 0.8)
    assert s1 == s2 == Fraction(3, 5) ** 2 * Fraction(7, 10) * Fraction(4, 5)
    # tie broken by lexicographic rank path
    assert ot._order_key(p1, s1) < ot._order_key(p2, s2)


def test_expected_accept_length_closed_form():
    # "Notes on Medusa", section 4: E[L] = sum over nodes of the path product.
    # For a full Cartesian tree (s1, s2): E = S1 + S1*S2 with S_k = sum_{r<s_k} a0 rho^r gamma^(k-1).
    s1, s2 = 3, 2
    t = ot.cartesian_tree((s1, s2))
    a0, rho, gamma = Fraction(3, 5), Fraction(7, 10), Fraction(4, 5)
    S1 = sum(a0 * rho ** r for r in range(s1))
    S2 = sum(a0 * rho ** r * gamma for r in range(s2))
    assert ot.expected_accept_length(t) == S1 + S1 * S2


def _prefix_relation(t):
    return [[t.paths[i][:len(t.paths[j])] == t.paths[j] for j in range(t.T)] for i in range(t.T)]


@pytest.mark.parametrize("maker", [lambda: ot.cartesian_tree((3, 2)), lambda: ot.cartesian_tree((2, 2, 2)),
                                   lambda: ot.scored_tree_greedy(4, 10, 64), lambda: ot.scored_tree_greedy(5, 16, 256)])
def test_mask_is_ancestor_or_self_relation(maker):
    # check (a): mask from parent walks == brute-force prefix relation of rank paths
    t = maker()
    M = ot.ancestor_mask(t)
    assert M == _prefix_relation(t)
    for i in range(t.T):
        assert sum(M[i]) == t.depth[i] + 1
        assert M[i][0] and M[i][i]
        for j in range(i + 1, t.T):
            assert not M[i][j]               # ancestors precede a node in the packing
    # two siblings' rows differ exactly in their own two bits
    for i in range(1, t.T):
        for j in range(i + 1, t.T):
            if t.parent[i] == t.parent[j]:
                diff = [c for c in range(t.T) if M[i][c] != M[j][c]]
                assert diff == [i, j]


def test_ancestors_listing():
    t = ot.cartesian_tree((2, 2))
    for i in range(t.T):
        a = ot.ancestors(t, i)
        assert a[0] == 0 and a[-1] == i and len(a) == t.depth[i] + 1
        assert [t.paths[j] for j in a] == [t.paths[i][:m] for m in range(t.depth[i] + 1)]


def test_workload_trees():
    from workloads import WORKLOADS
    assert ot.build_tree(WORKLOADS["tiny-fp32-T10"]).T == 10
    for name in ("7b-T64-L1024", "13b-T64-L4096"):
        assert ot.build_tree(WORKLOADS[name]).T == 64
    assert ot.build_tree(WORKLOADS["7b-B16-T42-paged"]).T == 42
    t = ot.build_tree(WORKLOADS["33b-B4-T256-L16384"])
    assert t.T == 256 and t.max_depth == 5      # 6-token accepted paths are reachable
