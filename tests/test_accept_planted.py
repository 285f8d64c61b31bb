"""Planted acceptance cases, checked on the CPU: the oracle's result on them covers what
the GPU test of the same cases claims to cover (every accepted length, passing edges
cut off by a failing ancestor, equal-depth ties), and typical edges sit far from their
thresholds.  Summary page, "Typical Acceptance Scheme" (longest accepted prefix over
all branches; the first token always accepted); "Notes on Medusa" section 3 (greedy walk).
"""

import functools

import pytest

from oracle import step as ostep
from oracle import tree as otree
from tests.planted import MARGIN, coverage, planted_case, typical_margin

# name -> ("cartesian", s) or ("scored", K, k, T): one to four 64-bit mask words
TREES = {
    "cart-3x2-T10": ("cartesian", (3, 2)),
    "7b-T64": ("scored", 4, 10, 64),
    "7b-T42": ("scored", 4, 10, 42),
    "T100": ("scored", 5, 16, 100),
    "T150": ("scored", 5, 16, 150),
    "33b-T256": ("scored", 5, 16, 256),
}

# (mode, tau, eps, delta)
MODES = {
    "greedy": ("greedy", 0.0, 0.09, 0.3),
    "typical-t0.7": ("typical", 0.7, 0.09, 0.3),
    "typical-t0": ("typical", 0.0, 0.09, 0.3),
    "typical-t1.3": ("typical", 1.3, 0.2, 0.5),
}


@functools.lru_cache(maxsize=None)
def oracle_tree(name):
    spec = TREES[name]
    return otree.cartesian_tree(spec[1]) if spec[0] == "cartesian" else otree.scored_tree_greedy(*spec[1:])


def batch_for(tree):
    return 3 * (tree.max_depth + 1)


@functools.lru_cache(maxsize=None)
def planted(tree_name, mode_name):
    t = oracle_tree(tree_name)
    mode, tau, eps, delta = MODES[mode_name]
    seed = 7000 + 31 * list(TREES).index(tree_name) + list(MODES).index(mode_name)
    case = planted_case(t.parent, t.depth, batch_for(t), mode, tau, eps, delta, seed)
    paths, n_acc = ostep.accept_path(case["stats_list"], case["edge"], case["tokens"], t, mode, eps, delta, tau)
    return case, paths, n_acc


@pytest.mark.parametrize("mode_name", list(MODES))
@pytest.mark.parametrize("tree_name", list(TREES))
def test_planted_cases_cover_the_rule(tree_name, mode_name):
    t = oracle_tree(tree_name)
    mode, tau, eps, delta = MODES[mode_name]
    case, paths, n_acc = planted(tree_name, mode_name)
    cov = coverage(case, n_acc, paths, t.parent, t.depth, mode, tau, eps, delta)
    assert cov["lengths"] == list(range(1, t.max_depth + 2))
    # each sequence lands exactly at the depth it aimed at
    assert [t.depth[x] + 1 for x in case["targets"]] == n_acc
    assert cov["cut"] >= 1
    if mode == "typical" and tau > 0:
        assert cov["ties"] >= 1
        assert typical_margin(case, t.parent, tau, eps, delta) >= MARGIN
    for b, p in enumerate(paths):
        assert p[0] == 0 and len(p) == n_acc[b]
