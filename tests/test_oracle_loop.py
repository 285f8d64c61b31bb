"""Pins of the oracle's chained steps (multi-step decoding), CPU only.

Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
Decoding Heads", section 3.2: the next iteration continues from the last accepted
token.  What the chain must satisfy, independently of how a step computes:
* a chain of one step is the step itself;
* each step's new prefix length is its prefix length plus its accepted count, and
  the next step starts from it;
* the next step's root token (the LM head's top token on the carried hidden state)
  is the argmax of the verifier row of the last accepted node: both are the LM head
  applied to the same vector;
* the cache keeps every earlier row and gains exactly the accepted path's rows.
"""

import json
import os

import numpy as np
import pytest

from oracle import find_seeds
from oracle import margins as om
from oracle import step as os_
from oracle import tree as ot
from workloads import make_inputs, step_qkv
from workloads.configs import get_case

SEEDS = json.load(open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "workloads", "seeds.json")))


def _loop(name, seed, steps, run_idx):
    w = get_case(name)
    inp = make_inputs(w, seed, steps=steps)
    qkv = [step_qkv(w, seed, s) for s in range(steps)]
    tree = ot.build_tree(w)
    run = w.accept[run_idx]
    return w, inp, qkv, tree, run, os_.decode_loop(w, inp, qkv, tree, run.mode, run.temperature, run.eps,
                                                    run.delta)


def test_step_qkv_zero_is_the_step_input():
    w = get_case("tiny-fp32-T10")
    a = make_inputs(w, 5)
    q0 = step_qkv(w, 5, 0)
    q1 = step_qkv(w, 5, 1)
    for n in ("q", "k", "v"):
        assert np.array_equal(q0[n], a[n])
        assert q1[n].shape == a[n].shape and not np.array_equal(q1[n], a[n])
    # more steps only add cache room
    b = make_inputs(w, 5, steps=4)
    assert b["Kc"].shape[1] == a["Kc"].shape[1] + 3 * (w.K + 1)
    assert np.array_equal(b["Kc"][:, :a["Kc"].shape[1]], a["Kc"])


@pytest.mark.parametrize("run_idx", [0, 1])
def test_one_step_chain_is_the_step(run_idx):
    w, inp, qkv, tree, run, res = _loop("tiny-fp32-T10", 1000, 1, run_idx)
    ref = os_.step(w, inp, tree, run.mode, run.temperature, run.eps, run.delta)
    assert res[0]["paths"] == ref["paths"] and res[0]["n_acc"] == ref["n_acc"]
    assert np.array_equal(res[0]["tokens"], ref["tokens"])
    assert np.array_equal(res[0]["o"], ref["o"])


@pytest.mark.parametrize("name,seed", [("tiny-fp32-T10", 1501), ("7b-mini", 6001), ("7b-B16-mini-paged", 8001)])
@pytest.mark.parametrize("run_idx", [0, 1])
def test_chain_invariants(name, seed, run_idx):
    steps = 3
    w, inp, qkv, tree, run, res = _loop(name, seed, steps, run_idx)
    T = tree.T
    lens = np.asarray(inp["prefix_len"], dtype=np.int64)
    pt = inp.get("page_table")
    prev_K = os_.to_f64(inp["Kc"])
    for s, r in enumerate(res):
        # prefix bookkeeping
        assert np.array_equal(np.asarray(r["new_len"]), lens + np.asarray(r["n_acc"]))
        assert np.array_equal(r["pos"][:, 0], lens)
        for b in range(w.B):
            last = r["paths"][b][-1]
            # the carried hidden state is the last accepted node's output ...
            if s + 1 < steps:
                # ... so the next root is that node's verifier argmax
                z_row = r["z"][b * T + last]
                assert res[s + 1]["tokens"][b, 0] == int(np.argmax(z_row))
            # cache: earlier rows unchanged, the path's rows appended
            L = int(lens[b])
            for j in range(L):
                if pt is None:
                    assert np.array_equal(r["K_new"][b, j], prev_K[b, j])
            for j, node in enumerate(r["paths"][b]):
                if pt is None:
                    assert np.array_equal(r["K_new"][b, L + j], r["k_rot"][b, node])
                else:
                    pg = pt[b, (L + j) // w.page_size]
                    assert np.array_equal(r["K_new"][pg, (L + j) % w.page_size], r["k_rot"][b, node])
        lens = np.asarray(r["new_len"], dtype=np.int64)
        prev_K = r["K_new"]


def test_stored_loop_seed_has_margin():
    """The seed stored for the three-step chain of the tiny case takes every decision
    of every step with margin >= MIN_MARGIN (re-checked from the oracle)."""
    rec = SEEDS["tiny-fp32-T10@loop3"]
    m = find_seeds.loop_margin(get_case("tiny-fp32-T10"), rec["seed"], 3)
    assert m >= om.MIN_MARGIN
    assert abs(m - rec["margin"]) < 1e-12
