"""The step at the full workload sizes, on the launch configuration bench.py times.

The oracle computes, at full size: every head logit (plain matrix products), the
top-k rows, the tree tokens, the rotated tree keys, the attention outputs of a sample
of heads (all nodes) and of a sample of nodes (all heads), and the verifier rows of
those sampled nodes.  Decisions are compared bit-exactly where the oracle's margin is
>= 1e-3 and checked for validity elsewhere.  Acceptance and compaction are checked by
properties that hold at any size: the path is the deepest node whose every edge
passes under the returned row statistics, and the cache rows are exact copies of the
path's rotated keys and values with every other row untouched.
"""

import functools
import math

import numpy as np
import pytest

from oracle import margins as om
from oracle import step as ostep
from oracle import tree as otree
from tests.parity_util import REL_TOL, SEEDS, note, rel_err_rows
from workloads import make_inputs
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu

FULL = ["7b-T64-L1024", "13b-T64-L4096", "7b-B16-T42-paged", "33b-B4-T256-L16384"]


def _seed(name):
    return SEEDS[name]["seed"] if name in SEEDS else 1000 * (list(WORKLOADS).index(name) + 1)


def _stats(a):
    import medusa_tree_verification_heads_amd as mdt
    return np.ascontiguousarray(a).view(mdt.ROW_STATS_DTYPE).reshape(-1)


def _passes(mode, tau, eps, delta, tok, st, edge):
    if mode == "greedy" or tau == 0.0:
        ok = tok == st["argmax"]
        return ok if mode == "greedy" else (ok and 1.0 > min(eps, delta)), math.inf
    lp = float(edge) / tau - float(st["logZ"])
    thr = min(math.log(eps), math.log(delta) - float(st["entropy"]))
    return lp > thr, abs(lp - thr)


@functools.lru_cache(maxsize=1)
def _workload_state(name):
    """Inputs and the oracle's head logits of one full-size workload (the runs of a workload
    share them; one workload is held at a time)."""
    w = WORKLOADS[name]
    seed = _seed(name)
    inp = make_inputs(w, seed)
    logits, _ = ostep.medusa_heads(inp["h"], inp["W1"], inp["W2"], inp["Wlm"])
    return w, seed, inp, logits


RUNS = [(n, i) for n in FULL for i in range(len(WORKLOADS[n].accept))]


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,run_idx", RUNS)
def test_full_size_step(name, run_idx):
    """Every acceptance run each workload names, at full size."""
    from medusa_tree_verification_heads_amd.step import VerifyStep
    w, seed, inp, logits = _workload_state(name)
    run = w.accept[run_idx]
    note(f"full size {name} seed {seed} run {run}")
    s = VerifyStep(w, inp, run.mode, run.temperature, run.eps, run.delta)
    s.run()
    g = s.outputs()
    del s
    tree = otree.build_tree(w)
    T, B, K1, k = tree.T, w.B, w.K + 1, w.k_cfg
    rng = np.random.default_rng(seed)

    # heads: all logits
    err = rel_err_rows(g["logits"], logits)
    note(f"{name}: heads rel err {err:.2e}")
    assert err <= REL_TOL

    # top-k per row: exact where every rank gap (through the k boundary) is >= 1e-3
    exact_rows = 0
    for b in range(B):
        for r in range(K1):
            ref_idx, ref_val = ostep.topk(logits[b, r], k)
            top = np.sort(logits[b, r])[::-1][:k + 1]
            if float(np.min(top[:-1] - top[1:])) >= om.MIN_MARGIN:
                assert g["topk_idx"][b, r].tolist() == ref_idx.tolist(), (b, r)
                exact_rows += 1
            else:   # every selected entry lies within 1e-3 of the true top-k
                assert np.all(logits[b, r, g["topk_idx"][b, r]] >= ref_val[-1] - om.MIN_MARGIN)
                assert len(set(g["topk_idx"][b, r].tolist())) == k
    note(f"{name}: top-k rows compared exactly {exact_rows}/{B * K1}")
    # tree tokens and positions follow the returned top-k
    for b in range(B):
        for i in range(T):
            assert g["tokens"][b, i] == g["topk_idx"][b, tree.depth[i], tree.rank[i]]
            assert g["pos"][b, i] == int(inp["prefix_len"][b]) + tree.depth[i]

    # attention: a sample of heads for every node, and every head for a sample of nodes
    heads = sorted(rng.choice(w.H, size=min(3, w.H), replace=False).tolist())
    nodes = sorted(set([0] + rng.choice(T, size=min(3, T - 1), replace=False).tolist()))
    pt = inp.get("page_table")
    oa, k_rot = ostep.tree_attention(inp["q"], inp["k"], inp["v"], inp["Kc"], inp["Vc"], inp["prefix_len"], tree,
                                     w.rope_theta, True, pt, w.page_size, heads=heads)
    ob, _ = ostep.tree_attention(inp["q"], inp["k"], inp["v"], inp["Kc"], inp["Vc"], inp["prefix_len"], tree,
                                 w.rope_theta, True, pt, w.page_size, queries=nodes)
    go = ostep.to_f64(g["o"])
    ea = rel_err_rows(go[:, :, heads], oa[:, :, heads])
    eb = rel_err_rows(go[:, nodes], ob[:, nodes])
    ek = rel_err_rows(ostep.to_f64(g["k_rot"]), k_rot)
    note(f"{name}: attention rel err (sampled heads {ea:.2e}, sampled nodes {eb:.2e}), k_rot {ek:.2e}")
    assert ea <= REL_TOL and eb <= REL_TOL and ek <= REL_TOL

    # verifier rows of the sampled nodes (oracle node outputs -> oracle logits)
    st = _stats(g["stats"])
    wlm = ostep.to_f64(inp["Wlm"])
    tau = run.temperature
    for b in range(B):
        for i in nodes:
            r = b * T + i
            z = wlm @ ob[b, i].reshape(-1)
            ref = ostep.row_stats(z, tau)
            scale = np.abs(z).max()
            assert abs(st["max"][r] - ref["max"]) <= REL_TOL * scale
            t2 = np.partition(z, -2)[-2:]
            if t2[1] - t2[0] >= om.MIN_MARGIN:
                assert st["argmax"][r] == ref["argmax"]
            if tau > 0:
                assert abs(st["logZ"][r] - ref["logZ"]) <= REL_TOL * abs(ref["logZ"])
                assert abs(st["entropy"][r] - ref["H"]) <= REL_TOL * max(abs(ref["H"]), 1e-3)
            for c in range(1, T):
                if tree.parent[c] == i:
                    assert abs(g["edge"][b, c] - z[g["tokens"][b, c]]) <= REL_TOL * scale

    # acceptance: the returned path is the deepest all-passing path under the returned statistics
    for b in range(B):
        ok = [True] * T
        tight = False
        for c in range(1, T):
            p, margin = _passes(run.mode, tau, run.eps, run.delta, int(g["tokens"][b, c]), st[b * T + tree.parent[c]],
                                g["edge"][b, c])
            ok[c] = bool(p)
            tight |= margin < 1e-4
        best = 0
        for c in range(1, T):
            if all(ok[j] for j in otree.ancestors(tree, c)) and tree.depth[c] > tree.depth[best]:
                best = c
        path = otree.ancestors(tree, best)
        if not tight:
            assert g["n_acc"][b] == len(path) and g["path"][b, :len(path)].tolist() == path
        assert g["path"][b, 0] == 0 and g["n_acc"][b] >= 1
    note(f"{name}: n_acc {g['n_acc'].tolist()[:8]}")

    # compaction: exact copies of the path rows, nothing else touched (sampled rows)
    L = inp["prefix_len"]
    touched = set()
    for b in range(B):
        for j in range(int(g["n_acc"][b])):
            node = int(g["path"][b, j])
            slot = int(L[b]) + j
            if pt is None:
                kk, vv = g["Kc"][b, slot], g["Vc"][b, slot]
                touched.add((b, slot))
            else:
                pg = pt[b, slot // w.page_size]
                kk, vv = g["Kc"][pg, slot % w.page_size], g["Vc"][pg, slot % w.page_size]
                touched.add((pg, slot % w.page_size))
            assert np.array_equal(kk, g["k_rot"][b, node]) and np.array_equal(vv, inp["v"][b, node])
        assert g["new_len"][b] == int(L[b]) + int(g["n_acc"][b])
    lead = g["Kc"].shape[:2]
    for _ in range(2000):
        a0, a1 = int(rng.integers(lead[0])), int(rng.integers(lead[1]))
        if (a0, a1) not in touched:
            assert np.array_equal(g["Kc"][a0, a1], inp["Kc"][a0, a1]) and np.array_equal(g["Vc"][a0, a1],
                                                                                        inp["Vc"][a0, a1])
