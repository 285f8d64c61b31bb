"""GPU parity of every call of the step against the CPU oracle (reduced sizes,
element by element, spanning several tiles with ragged tails).

End-to-end: the full GPU step on a workload's seeded inputs vs the oracle step.
Stage-wise: a call fed the oracle's inputs for that stage.
Integer/index outputs are compared bit-exactly (the seeds are chosen so that
every decision has margin >= 1e-3); floating outputs per row within 2e-2.
"""

import numpy as np
import pytest
import torch

from tests.parity_util import (REL_TOL, bf16_f64, cache_row, case_inputs, note, oracle_run, oracle_shared,
                               rel_err_rows, unique_rows)
from workloads.configs import PARITY_CASES

pytestmark = pytest.mark.gpu

CASES = list(PARITY_CASES)
RUNS = [(c, i) for c in CASES for i in range(len(PARITY_CASES[c].accept))]

_gpu_cache = {}


def gpu_step(name, run_idx):
    key = (name, run_idx)
    if key not in _gpu_cache:
        import medusa_tree_verification_heads_amd.step as st
        w, inp = case_inputs(name)
        run = w.accept[run_idx]
        note(f"gpu step {name} run={run}")
        s = st.VerifyStep(w, inp, run.mode, run.temperature, run.eps, run.delta, want_logits=True)
        s.run()
        _gpu_cache[key] = (s, s.outputs())
    return _gpu_cache[key]


def _stats_np(stats_i32):
    import medusa_tree_verification_heads_amd as mdt
    return np.ascontiguousarray(stats_i32).view(mdt.ROW_STATS_DTYPE).reshape(-1)


@pytest.mark.parametrize("name", CASES)
def test_heads(name):
    w, _ = case_inputs(name)
    _, g = gpu_step(name, 0)
    sh = oracle_shared(name)
    err = rel_err_rows(g["logits"], sh["logits"])
    note(f"{name} heads rel err {err:.2e}")
    assert err <= REL_TOL


@pytest.mark.parametrize("name", CASES)
def test_topk_tokens_positions(name):
    _, g = gpu_step(name, 0)
    sh = oracle_shared(name)
    assert np.array_equal(g["topk_idx"], sh["topk_idx"])
    assert rel_err_rows(g["topk_val"], sh["topk_val"]) <= REL_TOL
    assert np.array_equal(g["tokens"], sh["tokens"])
    assert np.array_equal(g["pos"], sh["pos"])


@pytest.mark.parametrize("name", CASES)
def test_tree_attention(name):
    w, _ = case_inputs(name)
    _, g = gpu_step(name, 0)
    sh = oracle_shared(name)
    go = bf16_f64(g["o"]) if w.dtype == "bf16" else g["o"]
    gk = bf16_f64(g["k_rot"]) if w.dtype == "bf16" else g["k_rot"]
    eo, ek = rel_err_rows(go, sh["o"]), rel_err_rows(gk, sh["k_rot"])
    exact = float(np.mean(gk == sh["k_rot"]))
    note(f"{name} attention o rel err {eo:.2e}, k_rot rel err {ek:.2e} (bit-equal fraction {exact:.6f})")
    assert eo <= REL_TOL and ek <= REL_TOL


@pytest.mark.parametrize("name,run_idx", RUNS)
def test_verify_logits(name, run_idx):
    w, _ = case_inputs(name)
    _, g = gpu_step(name, run_idx)
    sh, orr = oracle_shared(name), oracle_run(name, run_idx)
    tau = orr["run"].temperature
    z = sh["z"]
    assert rel_err_rows(g["vlogits"], z) <= REL_TOL
    st = _stats_np(g["stats"])
    scale = np.abs(z).max(axis=1)
    omax = np.array([s["max"] for s in orr["stats"]])
    assert np.all(np.abs(st["max"] - omax) <= REL_TOL * scale)
    uniq = unique_rows(z)
    for r in range(z.shape[0]):
        if r in uniq:
            assert st["argmax"][r] == orr["stats"][r]["argmax"], r
        else:   # near-tie: the chosen index must be a maximal value within the margin
            assert z[r, st["argmax"][r]] >= z[r].max() - 1e-3
    if tau > 0:
        oz = np.array([s["logZ"] for s in orr["stats"]])
        oh = np.array([s["H"] for s in orr["stats"]])
        assert np.all(np.abs(st["logZ"] - oz) <= REL_TOL * np.abs(oz))
        assert np.all(np.abs(st["entropy"] - oh) <= REL_TOL * np.maximum(np.abs(oh), 1e-3))
    e = g["edge"]
    assert np.all(e[:, 0] == 0)
    assert np.all(np.abs(e[:, 1:] - orr["edge"][:, 1:]) <= REL_TOL * scale.reshape(w.B, -1).max(axis=1, keepdims=True))


@pytest.mark.parametrize("name,run_idx", RUNS)
def test_accept_path(name, run_idx):
    _, g = gpu_step(name, run_idx)
    orr = oracle_run(name, run_idx)
    note(f"{name} run {run_idx}: n_acc gpu {g['n_acc'].tolist()} oracle {orr['n_acc']}")
    assert g["n_acc"].tolist() == orr["n_acc"]
    for b, p in enumerate(orr["paths"]):
        assert g["path"][b, :len(p)].tolist() == p
        assert np.all(g["path"][b, len(p):] == -1)


@pytest.mark.parametrize("name,run_idx", RUNS)
def test_kv_compact(name, run_idx):
    w, inp = case_inputs(name)
    _, g = gpu_step(name, run_idx)
    orr, sh = oracle_run(name, run_idx), oracle_shared(name)
    pt = inp.get("page_table")
    L = inp["prefix_len"]
    assert g["new_len"].tolist() == [int(L[b]) + n for b, n in enumerate(orr["n_acc"])]
    Kn, Vn = g["Kc"], g["Vc"]
    touched = set()
    for b in range(w.B):
        path = g["path"][b, :g["n_acc"][b]]
        for j, node in enumerate(path):
            slot = int(L[b]) + j
            # exact gather of the GPU's own rotated key / value rows
            assert np.array_equal(cache_row(Kn, b, slot, pt, w.page_size), g["k_rot"][b, node])
            assert np.array_equal(cache_row(Vn, b, slot, pt, w.page_size), inp["v"][b, node])
            # and within tolerance of the oracle's compacted key
            ok = sh["k_rot"][b, orr["paths"][b][j]]
            gk = cache_row(Kn, b, slot, pt, w.page_size)
            gk = bf16_f64(gk) if w.dtype == "bf16" else gk
            assert rel_err_rows(gk, ok) <= REL_TOL
            touched.add((b, slot))
    # every other cache row is unchanged
    if pt is None:
        mask = np.ones(Kn.shape[:2], dtype=bool)
        for b, s in touched:
            mask[b, s] = False
        assert np.array_equal(Kn[mask], inp["Kc"][mask]) and np.array_equal(Vn[mask], inp["Vc"][mask])
    else:
        mask = np.ones(Kn.shape[:2], dtype=bool)
        for b, s in touched:
            mask[pt[b, s // w.page_size], s % w.page_size] = False
        assert np.array_equal(Kn[mask], inp["Kc"][mask]) and np.array_equal(Vn[mask], inp["Vc"][mask])


# ---------------------------------------------------------------- stage-wise

@pytest.mark.parametrize("name", CASES)
def test_stage_topk_from_oracle_logits(name):
    import medusa_tree_verification_heads_amd as mdt
    from oracle import step as ostep
    w, inp = case_inputs(name)
    sh = oracle_shared(name)
    l32 = sh["logits"].astype(np.float32)
    tree = mdt.Tree.for_workload(w).to_device("cuda")
    pl = torch.from_numpy(inp["prefix_len"]).cuda()
    idx, val, tok, pos = mdt.topk_tree_expand(torch.from_numpy(l32).cuda(), w.k_cfg, tree, pl)
    torch.cuda.synchronize()
    ref = np.array([[ostep.topk(l32[b, r].astype(np.float64), w.k_cfg)[0] for r in range(w.K + 1)]
                    for b in range(w.B)])
    assert np.array_equal(idx.cpu().numpy(), ref)
    assert np.array_equal(val.cpu().numpy(), np.take_along_axis(l32, ref, axis=2))


def _tie_rows(V, rng):
    """Rows that stress the selection: coarse quantisation (ties at the top), all
    equal, three values only, -inf entries, the best values packed in one slice,
    and a row sorted in ascending order."""
    rows = [np.round(rng.standard_normal(V) * 4) / 4,
            np.zeros(V),
            rng.integers(0, 3, V).astype(np.float64),
            np.where(rng.random(V) < 0.5, -np.inf, rng.standard_normal(V)),
            np.concatenate([rng.standard_normal(max(V - 100, 0)) - 10, rng.standard_normal(min(V, 100))]),
            np.arange(V, dtype=np.float64)]
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("V,k", [(3001, 10), (32000, 10), (32000, 32), (32768, 32), (32769, 10), (50001, 16), (37, 32)])
def test_stage_topk_ties_and_fallback(V, k):
    """Exact order (value desc, index asc) on tie-heavy rows, including rows where
    far more elements than the survivor capacity reach the threshold."""
    import medusa_tree_verification_heads_amd as mdt
    from oracle import step as ostep
    note(f"topk ties V={V} k={k}")
    rng = np.random.default_rng(V * 100 + k)
    K = 4
    rows = _tie_rows(V, rng)
    B = 2
    logits = np.concatenate([rows, rows[::-1], rows[:-2] * -1.0])[: B * (K + 1)].reshape(B, K + 1, V)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    tree = mdt.Tree.scored(K, min(k, 10), 24).to_device("cuda")
    pl = torch.tensor([5, 9], dtype=torch.int32).cuda()
    idx, val, tok, pos = mdt.topk_tree_expand(torch.from_numpy(logits).cuda(), k, tree, pl)
    torch.cuda.synchronize()
    idx, val, tok = idx.cpu().numpy(), val.cpu().numpy(), tok.cpu().numpy()
    for b in range(B):
        for r in range(K + 1):
            ref_i, ref_v = ostep.topk(logits[b, r].astype(np.float64), k)
            assert idx[b, r].tolist() == ref_i.tolist(), (b, r)
            assert np.array_equal(val[b, r], logits[b, r, ref_i]), (b, r)
        t = tree.tree
        for i in range(t.T):
            assert tok[b, i] == idx[b, t.depth[i], t.rank[i]]


@pytest.mark.parametrize("V,tau", [(20000, 0.7), (32000, 0.0), (16500, 1.0)])
def test_verify_wide_vocabulary(V, tau):
    """One 64-row block over a vocabulary whose 64-column grid overfills the CUs (the
    128-column tile on 16 waves): full logits, row statistics and edge logits against the
    oracle's definitions, with a ragged last tile (20000, 16500)."""
    import medusa_tree_verification_heads_amd as mdt
    from oracle import step as ostep
    from oracle import tree as otree
    w = PARITY_CASES["7b-mini"]
    tree = otree.build_tree(w)
    dtree = mdt.Tree.for_workload(w).to_device("cuda")
    d, T = 256, tree.T
    rng = np.random.default_rng(V)
    x = ostep.round_bf16(rng.standard_normal((T, d)))
    W = ostep.round_bf16(rng.standard_normal((V, d)) * d ** -0.5)
    tok = rng.integers(0, V, (1, T))
    from workloads.gen import f32_to_bf16_bits
    xd = torch.from_numpy(f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    Wd = torch.from_numpy(f32_to_bf16_bits(W.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    stats, edge, logits = mdt.verify_logits(xd, Wd, dtree, torch.from_numpy(tok.astype(np.int32)).cuda(), tau,
                                            want_logits=True)
    torch.cuda.synchronize()
    z = x @ W.T
    assert rel_err_rows(logits.cpu().numpy(), z) <= REL_TOL
    st = _stats_np(stats.cpu().numpy())
    scale = np.abs(z).max(axis=1)
    for r in range(T):
        ref = ostep.row_stats(z[r], tau)
        assert abs(st["max"][r] - ref["max"]) <= REL_TOL * scale[r]
        t2 = np.partition(z[r], -2)[-2:]
        if t2[1] - t2[0] >= 1e-3:
            assert st["argmax"][r] == ref["argmax"], r
        if tau > 0:
            assert abs(st["logZ"][r] - ref["logZ"]) <= REL_TOL * abs(ref["logZ"])
            assert abs(st["entropy"][r] - ref["H"]) <= REL_TOL * max(abs(ref["H"]), 1e-3)
    e = edge.cpu().numpy()
    oe = ostep.edge_logits(z, tok, tree)
    assert np.all(e[:, 0] == 0) and np.all(np.abs(e - oe) <= REL_TOL * scale.max())


@pytest.mark.parametrize("name,run_idx", RUNS)
def test_stage_verify_accept_from_oracle_x(name, run_idx):
    import medusa_tree_verification_heads_amd as mdt
    w, inp = case_inputs(name)
    sh, orr = oracle_shared(name), oracle_run(name, run_idx)
    run = orr["run"]
    tree = mdt.Tree.for_workload(w).to_device("cuda")
    if w.dtype == "bf16":
        from workloads.gen import f32_to_bf16_bits
        xb = f32_to_bf16_bits(sh["x"].astype(np.float32))   # x is already bf16-valued
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        W = torch.from_numpy(inp["Wlm"].view(np.int16)).cuda().view(torch.bfloat16)
    else:
        x = torch.from_numpy(sh["x"].astype(np.float32)).cuda()
        W = torch.from_numpy(inp["Wlm"]).cuda()
    toks = torch.from_numpy(sh["tokens"].astype(np.int32)).cuda()
    stats, edge, _ = mdt.verify_logits(x, W, tree, toks, run.temperature)
    path, n = mdt.accept_path(stats, edge, toks, tree, mdt.GREEDY if run.mode == "greedy" else mdt.TYPICAL,
                              run.eps, run.delta, run.temperature)
    torch.cuda.synchronize()
    st = _stats_np(stats.cpu().numpy())
    uniq = unique_rows(sh["z"])
    for r in uniq:
        assert st["argmax"][r] == orr["stats"][r]["argmax"]
    assert n.cpu().numpy().tolist() == orr["n_acc"]
    for b, p in enumerate(orr["paths"]):
        assert path.cpu().numpy()[b, :len(p)].tolist() == p


@pytest.mark.parametrize("name", CASES)
def test_stage_compact_from_oracle_path(name):
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.step import to_device
    from workloads.gen import f32_to_bf16_bits
    w, inp = case_inputs(name)
    sh, orr = oracle_shared(name), oracle_run(name, 0)
    pt = inp.get("page_table")
    if w.dtype == "bf16":
        kr = f32_to_bf16_bits(sh["k_rot"].astype(np.float32))
    else:
        kr = sh["k_rot"].astype(np.float32)
    stride = max(len(p) for p in orr["paths"]) + 1
    path = np.full((w.B, stride), -1, dtype=np.int32)
    for b, p in enumerate(orr["paths"]):
        path[b, :len(p)] = p
    Kc, Vc = to_device(inp["Kc"].copy(), "cuda"), to_device(inp["Vc"].copy(), "cuda")
    cache = mdt.KVCache(Kc, Vc, None if pt is None else torch.from_numpy(pt).cuda(), w.page_size)
    new_len = mdt.kv_compact(torch.from_numpy(path).cuda(), torch.tensor(orr["n_acc"], dtype=torch.int32).cuda(),
                             to_device(kr, "cuda"), to_device(inp["v"], "cuda"), cache,
                             torch.from_numpy(inp["prefix_len"]).cuda())
    torch.cuda.synchronize()
    Kn = Kc.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else Kc.cpu().numpy()
    for b, p in enumerate(orr["paths"]):
        L = int(inp["prefix_len"][b])
        for j, node in enumerate(p):
            assert np.array_equal(cache_row(Kn, b, L + j, pt, w.page_size), kr[b, node])
    assert new_len.cpu().numpy().tolist() == [int(inp["prefix_len"][b]) + n for b, n in enumerate(orr["n_acc"])]


@pytest.mark.parametrize("T,d,V", [(1, 96, 1000), (17, 160, 5003), (64, 4128, 2048), (40, 128, 129), (64, 256, 32000)])
def test_verify_small_rows_ragged(T, d, V):
    """At most 64 node rows (one sequence's tree): inner dimensions that leave a partial
    last chunk (96, 160, 4128), a single row, vocabularies with ragged last tiles.  Full
    logits, row statistics and edge logits against the oracle's definitions."""
    import medusa_tree_verification_heads_amd as mdt
    from oracle import step as ostep
    from oracle import tree as otree
    from workloads.gen import f32_to_bf16_bits
    note(f"verify small rows T={T} d={d} V={V}")
    tree = otree.cartesian_tree(()) if T == 1 else otree.scored_tree_greedy(4, 10, T)
    dtree = (mdt.Tree.cartesian(()) if T == 1 else mdt.Tree.scored(4, 10, T)).to_device("cuda")
    rng = np.random.default_rng(T * 1000 + d)
    x = ostep.round_bf16(rng.standard_normal((T, d)))
    W = ostep.round_bf16(rng.standard_normal((V, d)) * d ** -0.5)
    tok = rng.integers(0, V, (1, T))
    xd = torch.from_numpy(f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    Wd = torch.from_numpy(f32_to_bf16_bits(W.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    for tau in (0.0, 0.7):
        stats, edge, logits = mdt.verify_logits(xd, Wd, dtree, torch.from_numpy(tok.astype(np.int32)).cuda(), tau,
                                                want_logits=True)
        torch.cuda.synchronize()
        z = x @ W.T
        assert rel_err_rows(logits.cpu().numpy(), z) <= REL_TOL
        st = _stats_np(stats.cpu().numpy())
        scale = np.abs(z).max(axis=1)
        for r in range(T):
            ref = ostep.row_stats(z[r], tau)
            assert abs(st["max"][r] - ref["max"]) <= REL_TOL * scale[r]
            t2 = np.partition(z[r], -2)[-2:]
            if t2[1] - t2[0] >= 1e-3:
                assert st["argmax"][r] == ref["argmax"], r
            if tau > 0:
                assert abs(st["logZ"][r] - ref["logZ"]) <= REL_TOL * abs(ref["logZ"])
                assert abs(st["entropy"][r] - ref["H"]) <= REL_TOL * max(abs(ref["H"]), 1e-3)
        e = edge.cpu().numpy()
        oe = ostep.edge_logits(z, tok, tree)
        assert np.all(e[:, 0] == 0) and np.all(np.abs(e - oe) <= REL_TOL * scale.max())


@pytest.mark.parametrize("B,T,d,V", [(16, 42, 256, 5003), (4, 160, 128, 1000), (6, 120, 128, 3000), (4, 256, 128, 2000), (4, 256, 192, 1900),
                                     (5, 220, 128, 777), (8, 160, 64, 32000)])
def test_verify_many_rows_ragged(B, T, d, V):
    """512 and more node rows (batches, large trees): 224 x 192 tiles (640 and 672 rows: three
    row blocks, the same as 256-row blocks, fewer padded rows), the 256 x 192 tile (720 rows),
    both with partials per 64 columns, and the 256 x 256 tile (1024 and more rows), with vocabularies
    whose last tile is partial or ends within its first pass (1900, 5003), a row count that
    leaves a partial last row block (1100), and a single 64-dim chunk.  Row statistics and
    edge logits against the oracle's definitions, per row."""
    import medusa_tree_verification_heads_amd as mdt
    from oracle import step as ostep
    from oracle import tree as otree
    from workloads.gen import f32_to_bf16_bits
    note(f"verify many rows B={B} T={T} d={d} V={V}")
    tree = otree.scored_tree_greedy(4, 10, T)
    dtree = mdt.Tree.scored(4, 10, T).to_device("cuda")
    M = B * T
    rng = np.random.default_rng(M + d + V)
    x = ostep.round_bf16(rng.standard_normal((M, d)))
    W = ostep.round_bf16(rng.standard_normal((V, d)) * d ** -0.5)
    tok = rng.integers(0, V, (B, T))
    xd = torch.from_numpy(f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    Wd = torch.from_numpy(f32_to_bf16_bits(W.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    z = x @ W.T
    scale = np.abs(z).max(axis=1)
    for tau in (0.0, 0.7):
        stats, edge, logits = mdt.verify_logits(xd, Wd, dtree, torch.from_numpy(tok.astype(np.int32)).cuda(), tau,
                                                want_logits=True)
        torch.cuda.synchronize()
        assert rel_err_rows(logits.cpu().numpy(), z) <= REL_TOL
        st = _stats_np(stats.cpu().numpy())
        for r in range(M):
            ref = ostep.row_stats(z[r], tau)
            assert abs(st["max"][r] - ref["max"]) <= REL_TOL * scale[r], r
            t2 = np.partition(z[r], -2)[-2:]
            if t2[1] - t2[0] >= 1e-3:
                assert st["argmax"][r] == ref["argmax"], r
            if tau > 0:
                assert abs(st["logZ"][r] - ref["logZ"]) <= REL_TOL * abs(ref["logZ"]), r
                assert abs(st["entropy"][r] - ref["H"]) <= REL_TOL * max(abs(ref["H"]), 1e-3), r
        e = edge.cpu().numpy()
        oe = ostep.edge_logits(z, tok, tree)
        assert np.all(e[:, 0] == 0) and np.all(np.abs(e - oe) <= REL_TOL * scale.max())
