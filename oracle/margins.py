"""Decision margins of a step, for the seed search and for parity tests.

Every discrete output of the step (top-k indices, the root token, greedy and
typical edge decisions, verifier argmaxes) is decided by comparing floating
point values.  Two correct implementations that round differently can only
disagree where the compared values are closer than their rounding error.  A
seed is accepted for bit-exact parity when every decision the step takes has
margin >= ``MIN_MARGIN`` (absolute, in logit or log-probability units), which
is orders of magnitude above float32 rounding of these quantities.

Decisions checked:
* each head row: gaps between consecutive ranks 0..k_cfg-1 and between rank
  k_cfg-1 and rank k_cfg (the inclusion boundary);
* greedy edges: |z'_p[x_c] - max_{v != x_c} z'_p[v]|;
* typical edges: |ln p(x_c) - ln min(eps, delta exp(-H_p))| (tau > 0).

Verifier rows whose top-1/top-2 gap is below the margin have an ambiguous
argmax; parity tests compare argmax only on rows returned by
``unique_argmax_rows`` and check validity elsewhere.
"""

from __future__ import annotations

import math

import numpy as np

MIN_MARGIN = 1e-3


def head_margin(logits: np.ndarray, k_cfg: int) -> float:
    """Smallest gap among the top k_cfg+1 sorted values of every head row."""
    B, K1, V = logits.shape
    m = math.inf
    for b in range(B):
        for r in range(K1):
            top = np.sort(logits[b, r])[::-1][:k_cfg + 1]
            if top.shape[0] > 1:
                m = min(m, float(np.min(top[:-1] - top[1:])))
    return m


def edge_margins(z, stats, tokens, tree, mode, eps, delta, tau):
    """Per-edge decision margins [B][T] (root column = inf)."""
    B, T = tokens.shape
    out = np.full((B, T), np.inf)
    for b in range(B):
        for c in range(1, T):
            r = b * T + tree.parent[c]
            row = z[r]
            x = int(tokens[b, c])
            if mode == "greedy" or tau == 0.0:
                others = np.delete(row, x)
                out[b, c] = abs(row[x] - others.max())
            else:
                st = stats[r]
                lp = row[x] / tau - st["logZ"]
                lthr = math.log(min(eps, delta * math.exp(-st["H"])))
                out[b, c] = abs(lp - lthr)
    return out


def unique_argmax_rows(z: np.ndarray, margin: float = MIN_MARGIN):
    """Rows whose largest value beats the second largest by at least ``margin``."""
    rows = []
    for r in range(z.shape[0]):
        if np.isnan(z[r]).any():
            continue
        t = np.partition(z[r], -2)[-2:]
        if t[1] - t[0] >= margin:
            rows.append(r)
    return rows


def step_margin(res: dict, w, tree, mode, eps, delta, tau) -> float:
    """Smallest margin over all decisions of one oracle step result."""
    m = head_margin(res["logits"], w.k_cfg)
    e = edge_margins(res["z"], res["stats"], res["tokens"], tree, mode, eps, delta, tau)
    return min(m, float(e.min()))


def rejection_margins(trace, B: int) -> np.ndarray:
    """Per sequence, the smallest margin of a rejection-sampling walk (``trace`` from
    ``step.accept_rejection``): |u - min(1, r/q)| of every tried child (inf when the
    acceptance probability is 1, since u < 1), and for the final draw the distance of
    u * total from the running sums around the chosen entry, relative to the total."""
    m = np.full(B, np.inf)
    for kind, b, u, val in trace:
        if kind == "accept":
            if val < 1.0:
                m[b] = min(m[b], abs(u - val))
        else:
            c = val
            t = u * c[-1]
            i = int(np.searchsorted(c, t, side="right"))
            lo = c[i - 1] if i > 0 else 0.0
            hi = c[min(i, c.shape[0] - 1)]
            m[b] = min(m[b], min(t - lo, hi - t) / c[-1])
    return m
