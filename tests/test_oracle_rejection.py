"""Pins of the oracle's rejection-sampling acceptance (CPU only).

Notes page, section 2 (and the summary page, "Typical Acceptance Scheme", first
paragraph): accepting a drafted x with probability min(1, p(x)/q(x)) and otherwise
drawing from norm(max(0, p - q)) makes the emitted token follow p exactly, for a
draft x ~ q.  With several candidates tried in turn (each rejection replacing the
target by the normalised residual), the emitted token still follows p when the
candidates are independent draws from q.  Both facts are checked on the oracle by
integrating over its random inputs (the uniforms are inputs, so every probability
is a measure of u values the oracle maps to an outcome), with nothing of the rule
re-typed in the test.
"""

import numpy as np
import pytest

from oracle import step as os_
from oracle.tree import _pack

G = 4000                       # grid points per uniform
GRID = (np.arange(G) + 0.5) / G


def _softmax(z, tau):
    e = np.exp(z / tau - (z / tau).max())
    return e / e.sum()


def _prob_accept(tree, z, hl, tokens, tau, child, others_reject=True):
    """Measure of u[child] for which the oracle accepts `child` (earlier siblings rejected)."""
    T = tree.T
    n = 0
    for u in GRID:
        ua = np.full((1, T), 1.0 - 1e-12)
        ua[0, child] = u
        paths, _, _ = os_.accept_rejection(z, hl, tokens, tree, tau, ua, np.array([0.5]))
        n += child in paths[0]
    return n / G


def _emit_dist(tree, z, hl, tokens, tau, V):
    """Distribution of the next token when every child is rejected (residual sampling)."""
    T = tree.T
    ua = np.full((1, T), 1.0 - 1e-12)
    cnt = np.zeros(V)
    for u in GRID:
        _, _, nxt = os_.accept_rejection(z, hl, tokens, tree, tau, ua, np.array([u]))
        if nxt[0] >= 0:
            cnt[nxt[0]] += 1
    return cnt / G


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_candidate_emits_target_distribution(seed):
    rng = np.random.default_rng(seed)
    V, tau = 5, 0.8
    tree = _pack([(), (0,)])
    z = rng.standard_normal((2, V)) * 1.5          # rows: root, child
    hl = rng.standard_normal((1, 2, V)) * 1.5      # head rows 0 (LM) and 1
    p = _softmax(z[0], tau)
    q = _softmax(hl[0, 1], tau)
    out = np.zeros(V)
    for x0 in range(V):                            # the draft token, drawn from q
        tokens = np.array([[0, x0]])
        a = _prob_accept(tree, z, hl, tokens, tau, 1)
        r = _emit_dist(tree, z, hl, tokens, tau, V)
        out += q[x0] * (a * np.eye(V)[x0] + (1 - a) * r)
    assert np.abs(out - p).max() < 3e-3


@pytest.mark.parametrize("seed", [3, 4])
def test_two_siblings_emit_target_distribution(seed):
    rng = np.random.default_rng(seed)
    V, tau = 4, 1.0
    tree = _pack([(), (0,), (1,)])
    z = rng.standard_normal((3, V)) * 1.5
    hl = rng.standard_normal((1, 2, V)) * 1.5
    p = _softmax(z[0], tau)
    q = _softmax(hl[0, 1], tau)
    out = np.zeros(V)
    for x1 in range(V):
        for x2 in range(V):                        # independent draws from q
            tokens = np.array([[0, x1, x2]])
            a1 = _prob_accept(tree, z, hl, tokens, tau, 1)
            # child 2 is tried only after child 1 is rejected
            T = tree.T
            n2 = 0
            for u in GRID:
                ua = np.array([[1.0, 1.0 - 1e-12, u]])
                paths, _, _ = os_.accept_rejection(z, hl, tokens, tree, tau, ua, np.array([0.5]))
                n2 += 2 in paths[0]
            a2 = n2 / G
            r2 = _emit_dist(tree, z, hl, tokens, tau, V)
            e = a1 * np.eye(V)[x1] + (1 - a1) * (a2 * np.eye(V)[x2] + (1 - a2) * r2)
            out += q[x1] * q[x2] * e
    assert np.abs(out - p).max() < 5e-3


def test_identical_draft_and_target_accept_every_first_child():
    rng = np.random.default_rng(7)
    V, tau = 6, 0.7
    tree = _pack([(), (0,), (1,), (0, 0), (0, 1), (1, 0)])
    row = rng.standard_normal(V)
    z = np.tile(row, (tree.T, 1))
    hl = np.tile(row, (1, 3, 1))
    tokens = rng.integers(0, V, (1, tree.T))
    ua = rng.uniform(0, 1 - 1e-9, (1, tree.T))
    paths, n_acc, _ = os_.accept_rejection(z, hl, tokens, tree, tau, ua, np.array([0.3]))
    # p == q: every first child passes (acceptance probability 1), down to a leaf
    assert paths[0] == [0, 1, 3] and n_acc == [3]


def test_rejected_mass_and_root():
    V, tau = 3, 1.0
    tree = _pack([(), (0,)])
    z = np.array([[0.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    hl = np.array([[[0.0, 0.0, 0.0], [50.0, 0.0, 0.0]]])  # q puts all mass on token 0
    tokens = np.array([[0, 0]])
    # p(0)/q(0) = 1/3: u = 0.3 accepts, u = 0.4 rejects
    p1, _, _ = os_.accept_rejection(z, hl, tokens, tree, tau, np.array([[0.0, 0.3]]), np.array([0.0]))
    p2, n2, nx = os_.accept_rejection(z, hl, tokens, tree, tau, np.array([[0.0, 0.4]]), np.array([0.0]))
    assert p1[0] == [0, 1] and p2[0] == [0] and n2 == [1]
    # residual max(0, p - q) has no mass on token 0: the lowest u draws token 1
    assert nx == [1]
