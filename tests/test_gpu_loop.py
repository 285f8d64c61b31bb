"""Chained steps on the GPU (multi-step decoding) against the oracle.

* The tiny fp32 case has a seed whose three-step chain takes every decision with
  margin >= 1e-3 (``tiny-fp32-T10@loop3`` in workloads/seeds.json): the GPU chain is
  compared with the oracle chain, integers bit-exactly.
* Larger cases: after the first step the carried hidden states are attention outputs,
  whose logits lie close together, so a chain may legitimately leave the oracle's
  chain at a near-tie.  The GPU chain is compared with the oracle chain (both started
  from the drawn inputs; the oracle never sees a GPU value) step by step while the two
  agree: head logits and node outputs within the tolerance, top-k rows exactly where
  the oracle's gaps exceed twice the observed logit difference, accepted paths exactly
  where every edge margin is >= 1e-3.  Once a step's candidates differ, later steps are
  checked by properties of the GPU's own values only (top-k of its logits, tree tokens
  of its top-k, positions, path structure, the carried row).
* A chain equals independent single steps started from the chain's states.
"""

import numpy as np
import pytest
import torch

from oracle import margins as om
from oracle import step as ostep
from oracle import tree as otree
from tests.parity_util import REL_TOL, SEEDS, bf16_f64, clear_topk_rows, exact_topk, note, rel_err_rows
from workloads import make_inputs, step_qkv
from workloads.configs import get_case

pytestmark = pytest.mark.gpu

STEPS = 3


def _host(x):
    torch.cuda.synchronize()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def _make(name, seed, run_idx, want_logits=False, reuse=True):
    from medusa_tree_verification_heads_amd.step import DecodeLoop
    w = get_case(name)
    inp = make_inputs(w, seed, steps=STEPS)
    qkv = [step_qkv(w, seed, s) for s in range(STEPS)]
    run = w.accept[min(run_idx, len(w.accept) - 1)]
    note(f"loop {name} seed {seed} {run}")
    loop = DecodeLoop(w, inp, qkv, run.mode, run.temperature, run.eps, run.delta, want_logits=want_logits,
                      reuse_lm_head=reuse)
    return w, inp, qkv, run, loop


@pytest.mark.parametrize("reuse", [True, False])
@pytest.mark.parametrize("run_idx", [0, 1])
def test_tiny_chain_matches_oracle_chain(run_idx, reuse):
    seed = SEEDS["tiny-fp32-T10@loop3"]["seed"]
    w, inp, qkv, run, loop = _make("tiny-fp32-T10", seed, run_idx, reuse=reuse)
    loop.run()
    tree = otree.build_tree(w)
    ref = ostep.decode_loop(w, inp, qkv, tree, run.mode, run.temperature, run.eps, run.delta)
    tokens, paths, n_acc = _host(loop.tokens), _host(loop.paths), _host(loop.n_acc)
    for s, r in enumerate(ref):
        assert np.array_equal(tokens[s], r["tokens"]), s
        assert n_acc[s].tolist() == r["n_acc"], s
        for b in range(w.B):
            assert paths[s, b, :n_acc[s, b]].tolist() == r["paths"][b], (s, b)
        assert _host(loop.lens[s + 1]).tolist() == list(r["new_len"]), s
        if s + 1 < STEPS:
            hn = _host(loop.h[s + 1]).astype(np.float64)
            href = np.stack([r["o"][b, r["paths"][b][-1]].reshape(w.d) for b in range(w.B)])
            assert rel_err_rows(hn, href) <= REL_TOL, s
    Kc = _host(loop.step.t["Kc"]).astype(np.float64)
    assert rel_err_rows(Kc.reshape(-1, w.H * w.Dh), ref[-1]["K_new"].reshape(-1, w.H * w.Dh)) <= REL_TOL


@pytest.mark.parametrize("run_idx", [0, 1])
@pytest.mark.parametrize("name", ["7b-mini", "7b-B16-mini-paged", "33b-mini"])
def test_chain_against_oracle_chain(name, run_idx):
    seed = SEEDS[name]["seed"]
    w, inp, qkv, run, loop = _make(name, seed, run_idx, want_logits=True)
    st = loop.step
    tree = otree.build_tree(w)
    T, B = tree.T, w.B
    ref = ostep.decode_loop(w, inp, qkv, tree, run.mode, run.temperature, run.eps, run.delta)
    together, compared = True, 0
    for s in range(STEPS):
        L = _host(loop.lens[s]).astype(np.int32)
        loop.run_step(s)
        logits = _host(st.logits)
        topk = _host(st.topk_idx)
        tokens = _host(loop.tokens[s])
        pos = _host(st.pos)
        n_acc = _host(loop.n_acc[s])
        paths = _host(loop.paths[s])
        hn = _host(loop.h[s + 1])
        o_bits = _host(st.o).reshape(B, T, w.d)
        # properties of the GPU's own values, at every step
        for b in range(B):
            for k in range(w.K + 1):
                assert topk[b, k].tolist() == exact_topk(logits[b, k], w.k_cfg).tolist(), (s, b, k)
        for i in range(T):
            assert np.array_equal(tokens[:, i], topk[:, tree.depth[i], tree.rank[i]]), (s, i)
            assert np.array_equal(pos[:, i], L + tree.depth[i]), (s, i)
        assert np.array_equal(_host(loop.lens[s + 1]), L + n_acc), s
        for b in range(B):
            path = paths[b, :n_acc[b]].tolist()
            assert path[0] == 0 and all(tree.parent[path[j]] == path[j - 1] for j in range(1, len(path))), (s, b)
            assert np.array_equal(hn[b], o_bits[b, path[-1]]), (s, b)
        if not together:
            continue
        # the oracle chain, while the two chains agree
        r = ref[s]
        assert rel_err_rows(logits, r["logits"]) <= REL_TOL, s
        o = bf16_f64(_host(st.o)) if w.dtype == "bf16" else _host(st.o).astype(np.float64)
        assert rel_err_rows(o.reshape(-1, w.Dh), r["o"].reshape(-1, w.Dh)) <= REL_TOL, s
        diff = np.abs(logits.astype(np.float64) - r["logits"]).max(axis=-1)
        clear = clear_topk_rows(r["logits"], diff, w.k_cfg)
        for b in range(B):
            for k in range(w.K + 1):
                if clear[b, k]:
                    assert topk[b, k].tolist() == r["topk_idx"][b, k].tolist(), (s, b, k)
        if not np.array_equal(tokens, r["tokens"]):
            note(f"{name} step {s}: candidates differ at a near-tie; the chains part")
            together = False
            continue
        em = om.edge_margins(r["z"], r["stats"], r["tokens"], tree, run.mode, run.eps, run.delta, run.temperature)
        dz = np.abs(_host(st.vlogits).astype(np.float64) - r["z"]).reshape(B, -1).max(axis=1)
        for b in range(B):
            # an edge test moves by at most 2|dz| (greedy) or 4|dz|/tau (typical, log-prob units)
            need = max(om.MIN_MARGIN, 4 * dz[b] / (run.temperature or 0.5))
            if np.array_equal(tokens[b], r["tokens"][b]) and em[b].min() >= need:
                assert paths[b, :n_acc[b]].tolist() == r["paths"][b], (s, b)
                compared += 1
        together = n_acc.tolist() == r["n_acc"] and all(
            paths[b, :n_acc[b]].tolist() == r["paths"][b] for b in range(B))
        note(f"{name} step {s}: {int(clear.sum())} of {clear.size} top-k rows clear; chains agree: {together}")
    note(f"{name}: accepted paths compared on {compared} of {STEPS * B} sequence-steps")
    assert compared >= 1


@pytest.mark.parametrize("name", ["7b-mini", "7b-B16-mini-paged"])
def test_chain_equals_independent_steps(name):
    from medusa_tree_verification_heads_amd.step import VerifyStep
    seed = SEEDS[name]["seed"]
    # without the LM-head reuse: every step is then exactly the single step (with it, the
    # LM-head slot comes from the verifier's fp32 sums instead of the head GEMV's)
    w, inp, qkv, run, loop = _make(name, seed, 1, reuse=False)
    for s in range(STEPS):
        state = dict(inp)
        state.update(qkv[s])
        state["h"] = _host(loop.h[s])
        state["Kc"], state["Vc"] = _host(loop.step.t["Kc"]), _host(loop.step.t["Vc"])
        state["prefix_len"] = _host(loop.lens[s]).astype(np.int32)
        single = VerifyStep(w, state, run.mode, run.temperature, run.eps, run.delta)
        single.run()
        one = single.outputs()
        loop.run_step(s)
        assert np.array_equal(one["tokens"], _host(loop.tokens[s])), s
        assert np.array_equal(one["n_acc"], _host(loop.n_acc[s])), s
        assert np.array_equal(one["new_len"], _host(loop.lens[s + 1])), s
        assert np.array_equal(one["Kc"], _host(loop.step.t["Kc"])), s
        assert np.array_equal(one["o"], _host(loop.step.o)), s


def test_chain_repeats_and_replays_as_graph():
    name = "7b-mini"
    w, inp, qkv, run, loop = _make(name, SEEDS[name]["seed"], 1)
    loop.run()
    first = [_host(x) for x in (loop.tokens, loop.paths, loop.n_acc, loop.lens[STEPS], loop.h[STEPS])]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        loop.run()
    for _ in range(3):
        g.replay()
        again = [_host(x) for x in (loop.tokens, loop.paths, loop.n_acc, loop.lens[STEPS], loop.h[STEPS])]
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
        loop.run()
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["7b-mini", "7b-B16-mini-paged"])
def test_reused_lm_head_slot(name):
    """With the LM-head reuse, step s >= 1's slot 0 is bit for bit step s-1's verifier row
    of each sequence's deepest accepted node, the other slots are the heads of the carried
    hidden state, and the root token is that row's top token."""
    import medusa_tree_verification_heads_amd as mdt
    w, inp, qkv, run, loop = _make(name, SEEDS[name]["seed"], 1)
    st = loop.step
    T = st.tree.T
    prev = None
    for s in range(STEPS):
        loop.run_step(s)
        logits = _host(st.logits)
        if prev is not None:
            z, paths, n_acc = prev
            for b in range(w.B):
                last = paths[b, n_acc[b] - 1]
                assert np.array_equal(logits[b, 0], z[b * T + last]), (s, b)
                assert _host(loop.tokens[s])[b, 0] == exact_topk(z[b * T + last], 1)[0]
            # slots 1..K: the heads on the carried state, as a fresh heads call computes them
            ref = mdt.medusa_heads(loop.h[s], st.t["W1"], st.t["W2"], st.t["Wlm"])
            assert np.array_equal(logits[:, 1:], _host(ref)[:, 1:]), s
        prev = (_host(loop.vlogits), _host(loop.paths[s]), _host(loop.n_acc[s]))



def test_next_logits_rows_and_invalid_sequences():
    """mdt_next_logits copies each sequence's last accepted node's verifier row into slot 0
    exactly, leaves slots 1..K alone, and writes zeros for a sequence whose n_acc or last
    path node is out of range."""
    import medusa_tree_verification_heads_amd as mdt
    B, T, V, K, stride = 4, 10, 3001, 3, 4
    g = torch.Generator(device="cuda").manual_seed(5)
    z = torch.randn((B * T, V), device="cuda", generator=g)
    head = torch.full((B, K + 1, V), 9.0, device="cuda")
    path = torch.tensor([[0, 2, 5, -1], [0, 1, -1, -1], [0, 3, 7, 9], [0, 12, -1, -1]], dtype=torch.int32,
                        device="cuda")
    n_acc = torch.tensor([3, 0, 4, 2], dtype=torch.int32, device="cuda")   # b=1: n_acc 0; b=3: node 12 >= T
    mdt.next_logits(z, path, n_acc, head)
    zh, hh = _host(z), _host(head)
    assert np.array_equal(hh[0, 0], zh[0 * T + 5]) and np.array_equal(hh[2, 0], zh[2 * T + 9])
    assert np.all(hh[1, 0] == 0) and np.all(hh[3, 0] == 0)
    assert np.all(hh[:, 1:] == 9.0)
