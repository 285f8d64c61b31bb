"""A step on a tree built from an accuracy table (mdt_tree_build_table): tree tokens,
positions and tree attention against the oracle on the same table tree."""

import numpy as np
import pytest

from oracle import step as ostep
from oracle import tree as otree
from tests.parity_util import REL_TOL, bf16_f64, case_inputs, note, oracle_shared, rel_err_rows, seed_of
from workloads import make_inputs
from workloads.configs import scaled

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [16, 48, 100])
def test_step_on_table_tree(T):
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.step import VerifyStep
    name = "7b-mini"
    w, inp = case_inputs(name)
    rng = np.random.default_rng(T)
    acc = np.ascontiguousarray(np.sort(rng.uniform(0.01, 0.6, (w.K, w.k_cfg)), axis=1)[:, ::-1])
    ltree = mdt.Tree.from_table(acc, T)
    otr = otree.table_tree_greedy(w.K, w.k_cfg, T, acc)
    note(f"table tree T={T} depth {otr.max_depth}")
    # the same weights, h and cache; the tree's q/k/v drawn for T nodes
    inp = make_inputs(scaled(w, T=T), seed_of(name))
    st = VerifyStep(w, inp, "typical", 0.7, tree=ltree)
    st.run()
    g = st.outputs()
    sh = oracle_shared(name)
    tokens, pos = ostep.tree_expand(sh["topk_idx"], otr, inp["prefix_len"])
    assert np.array_equal(g["tokens"], tokens)
    assert np.array_equal(g["pos"], pos)
    o, k_rot = ostep.tree_attention(inp["q"], inp["k"], inp["v"], inp["Kc"], inp["Vc"],
                                    inp["prefix_len"], otr, w.rope_theta, bf16_store=True)
    assert rel_err_rows(bf16_f64(g["o"]).reshape(-1, w.Dh), o.reshape(-1, w.Dh)) <= REL_TOL
