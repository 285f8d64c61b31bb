"""Pins of the full-forward oracle (``oracle/forward.py``) to facts other than itself.

* RMSNorm: a constant row c gives c / sqrt(c^2 + eps) * g; with eps = 0 the result
  does not change when the row is scaled by a power of two (exactly).
* SiLU-gated product: silu(0) = 0, silu(1) = 1 / (1 + 1/e), silu(u) -> u for large u
  and -> 0 for very negative u.
* A decoder layer whose output and down projections are zero is the identity (the
  residual wiring), and with a one-node tree over an empty prefix the attention
  returns v itself (softmax over a single key), so the layer adds exactly v Wo^T.
* Tree attention through a stack of layers: every node's output equals the output
  of its root path run through the same layers as a plain chain (causal attention),
  the whole-model form of the single-layer per-path check.  A wrong mask, position
  or layer order breaks this at O(1).
* Chained forward steps (summary page, section 3.2: the next iteration continues from
  the last accepted token): a one-step chain is the forward step; each step's new
  length is its length plus its accepted count and the next step's positions start
  there; the next root token (LM head on the carried row) is the argmax of the
  verifier row of the last accepted node, since both apply W_lm to the same vector;
  every layer's cache keeps its earlier rows and gains exactly that layer's keys and
  values of the accepted path.
* The interleaved gate/up layout of the library's SwiGLU product is a row
  permutation of [Wg; Wu] with the stated pattern (host-side logic).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import find_seeds
from oracle import forward as ofw
from oracle import step as ostep
from oracle import tree as otree
from workloads.configs import FORWARD_CASES, scaled
from workloads import make_inputs
from workloads.gen import forward_inputs, layer_inputs


def test_rmsnorm_constant_row():
    for c in (0.5, -3.0, 7.25):
        x = np.full((1, 64), c)
        g = ostep.round_bf16(np.linspace(0.5, 1.5, 64))
        for eps in (0.0, 1e-6, 0.25):
            y = ofw.rmsnorm(x, g, eps)
            want = ostep.round_bf16(c / math.sqrt(c * c + eps) * g)
            assert np.array_equal(y[0], want)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(3)
    x = ostep.round_bf16(rng.standard_normal((5, 96)))
    g = ostep.round_bf16(1 + 0.1 * rng.standard_normal(96))
    y = ofw.rmsnorm(x, g, 0.0)
    assert np.array_equal(ofw.rmsnorm(4.0 * x, g, 0.0), y)
    assert np.array_equal(ofw.rmsnorm(x / 8.0, g, 0.0), y)
    # unit root mean square before the gain
    z = ofw.rmsnorm(x, np.ones(96), 0.0)
    assert np.allclose(np.sqrt(np.mean(z * z, axis=1)), 1.0, atol=1e-2)


def test_swiglu_values():
    assert ofw.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0
    assert ofw.swiglu(np.array([1.0]), np.array([1.0]))[0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    assert ofw.swiglu(np.array([40.0]), np.array([2.0]))[0] == pytest.approx(80.0, rel=1e-15)
    assert abs(ofw.swiglu(np.array([-40.0]), np.array([2.0]))[0]) < 1e-15


def _mini():
    return FORWARD_CASES["7b-mini-x2"]


def test_layer_identity_without_output_projections():
    dw = _mini()
    w = dw.base
    lw = dict(layer_inputs(dw, 5, 0))
    lw["Wo"] = np.zeros_like(lw["Wo"])
    lw["Wd"] = np.zeros_like(lw["Wd"])
    tree = otree.build_tree(w)
    rng = np.random.default_rng(1)
    x = ostep.round_bf16(rng.standard_normal((tree.T, w.d)))
    y, _, _ = ofw.decoder_layer(x, lw, np.array([w.L], dtype=np.int32), tree, w, dw.norm_eps)
    assert np.array_equal(y, x)


def test_single_key_attention_adds_v():
    dw = _mini()
    w = scaled(dw.base, name="mini-L0", L=0)
    lw = dict(layer_inputs(dw, 6, 0))
    lw["Wd"] = np.zeros_like(lw["Wd"])
    lw["Kc"] = lw["Kc"][:, :1] * 0
    lw["Vc"] = lw["Vc"][:, :1] * 0
    tree = otree.cartesian_tree(())
    assert tree.T == 1
    rng = np.random.default_rng(2)
    x = ostep.round_bf16(rng.standard_normal((1, w.d)))
    y, _, v = ofw.decoder_layer(x, lw, np.array([0], dtype=np.int32), tree, w, dw.norm_eps)
    h = ofw.rmsnorm(x, ostep.to_f64(lw["g_attn"]), dw.norm_eps)
    v_direct = ostep.round_bf16(h @ ostep.to_f64(lw["Wv"]).T)
    assert np.array_equal(v.reshape(1, w.d), v_direct)
    want = ostep.round_bf16(x + v_direct @ ostep.to_f64(lw["Wo"]).T)
    assert np.array_equal(y, want)


def _run_layers(dw, x, layers, tree, prefix_len):
    for lw in layers:
        x, _, _ = ofw.decoder_layer(x, lw, prefix_len, tree, dw.base, dw.norm_eps)
    return x


@pytest.mark.parametrize("node", [0, 5, 23, 63])
def test_tree_forward_equals_path_chains(node):
    dw = _mini()
    w = dw.base
    seed = 11
    layers = [layer_inputs(dw, seed, l) for l in range(dw.n_layers)]
    E = ostep.to_f64(forward_inputs(dw, seed)["E"])
    tree = otree.build_tree(w)
    rng = np.random.default_rng(4)
    tokens = rng.integers(0, w.V, tree.T)
    L = np.array([w.L], dtype=np.int32)
    x_tree = _run_layers(dw, E[tokens], layers, tree, L)
    path = otree.ancestors(tree, node)
    chain = otree.cartesian_tree((1,) * (len(path) - 1))
    x_chain = _run_layers(dw, E[tokens[path]], layers, chain, L)
    a, b = x_tree[node], x_chain[-1]
    scale = np.abs(b).max()
    # identical arithmetic up to summation order: a handful of bf16 roundings may land
    # one unit apart, far below what a wrong mask, position or layer order produces
    assert np.abs(a - b).max() <= 2e-2 * scale
    assert np.mean(a == b) > 0.9


def _chain(name, seed, steps, run_idx):
    dw = FORWARD_CASES[name]
    w = dw.base
    inp = make_inputs(w, seed, parts=("h", "W1", "W2", "Wlm"), steps=steps)
    fin = forward_inputs(dw, seed)
    layers = [layer_inputs(dw, seed, l, steps=steps) for l in range(dw.n_layers)]
    tree = otree.build_tree(w)
    run = w.accept[run_idx]
    res = ofw.forward_loop(dw, inp, fin, layers, tree, steps, run.mode, run.temperature, run.eps, run.delta)
    return dw, inp, fin, layers, tree, run, res


@pytest.mark.parametrize("run_idx", [0, 1])
def test_one_step_forward_chain_is_the_forward(run_idx):
    dw, inp, fin, layers, tree, run, res = _chain("7b-mini-x2", 21, 1, run_idx)
    ref = ofw.forward(dw, inp, fin, layers, tree, run.mode, run.temperature, run.eps, run.delta)
    assert res[0]["paths"] == ref["paths"] and res[0]["n_acc"] == ref["n_acc"]
    assert np.array_equal(res[0]["tokens"], ref["tokens"]) and np.array_equal(res[0]["xf"], ref["xf"])


@pytest.mark.parametrize("run_idx", [0, 1])
def test_forward_chain_invariants(run_idx):
    steps = 3
    dw, inp, fin, layers, tree, run, res = _chain("7b-mini-B2-x2", 23, steps, run_idx)
    w, T = dw.base, tree.T
    lens = np.asarray(inp["prefix_len"], dtype=np.int64)
    prev = [(ostep.to_f64(lw["Kc"]), ostep.to_f64(lw["Vc"])) for lw in layers]
    for s, r in enumerate(res):
        assert np.array_equal(np.asarray(r["new_len"]), lens + np.asarray(r["n_acc"]))
        assert np.array_equal(r["pos"][:, 0], lens)
        for b in range(w.B):
            last = r["paths"][b][-1]
            if s + 1 < steps:
                assert res[s + 1]["tokens"][b, 0] == int(np.argmax(r["z"][b * T + last]))
            L = int(lens[b])
            for l, (Kn, Vn) in enumerate(r["caches"]):
                Kp, Vp = prev[l]
                assert np.array_equal(Kn[b, :L], Kp[b, :L]) and np.array_equal(Vn[b, :L], Vp[b, :L])
                for j, node in enumerate(r["paths"][b]):
                    assert np.array_equal(Kn[b, L + j], r["k_rot"][l][b, node])
                    assert np.array_equal(Vn[b, L + j], r["v"][l][b, node])
                n = len(r["paths"][b])
                assert np.array_equal(Kn[b, L + n:], Kp[b, L + n:])
        lens = lens + np.asarray(r["n_acc"])
        prev = r["caches"]


@pytest.mark.parametrize("name", ["7b-mini-x2", "7b-mini-B2-x2"])
def test_stored_forward_loop_seed_has_margin(name):
    """The stored three-step forward-chain seeds pass their margin rule (re-checked)."""
    seeds = json.load(open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "workloads", "seeds.json")))
    rec = seeds[f"fwd:{name}@loop3"]
    m = find_seeds.forward_margin(FORWARD_CASES[name], rec["seed"], 3)
    assert m >= 1.0 and abs(m - rec["margin"]) < 1e-12


def test_interleave_gate_up_layout():
    torch = pytest.importorskip("torch")
    from medusa_tree_verification_heads_amd import interleave_gate_up
    F, K = 48, 8
    Wg = torch.arange(F * K, dtype=torch.float32).reshape(F, K)
    Wu = -Wg - 1
    W = interleave_gate_up(Wg, Wu)
    assert W.shape == (2 * F, K)
    for i in range(F // 16):
        for c in range(16):
            assert torch.equal(W[32 * i + c], Wg[16 * i + c])
            assert torch.equal(W[32 * i + 16 + c], Wu[16 * i + c])
