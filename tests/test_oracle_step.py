"""Pins of the oracle's step functions against the pages, closed forms, library
routines and brute force (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import step as os_
from oracle import tree as ot
from oracle import margins as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- storage format

def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # exact ties: bf16 value + half an ulp (both parities of the kept bit)
    base = torch.tensor(rng.standard_normal(200), dtype=torch.float32).to(torch.bfloat16).float().numpy()
    ulp = 2.0 ** (np.floor(np.log2(np.abs(base))) - 7)      # bf16 spacing at base
    ties = np.concatenate([base + ulp / 2, base - ulp / 2]).astype(np.float32)
    x32 = np.concatenate([x32, ties, np.float32([0.0, -0.0, 1.0, -3.5])])
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    got = os_.round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]        # skip inf/nan patterns
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(os_.bf16_to_f64(bits), ref)


# ---------------------------------------------------------------- heads

def test_silu_closed_form():
    assert os_.silu(np.array([0.0]))[0] == 0.0
    assert abs(os_.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(os_.silu(np.array([-1.0]))[0] - (-0.2689414213699951)) < 1e-16


def test_heads_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "heads_hand.json")))
    logits, a = os_.medusa_heads(np.array([g["h"]]), np.array(g["W1"]), np.array(g["W2"]), np.array(g["Wlm"]))
    np.testing.assert_allclose(logits, np.array(g["logits"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(a, np.array(g["a"]), rtol=0, atol=1e-15)


def test_heads_at_init_equal_lm_head():
    # summary page, "MEDUSA Heads": with W1 = 0 and W2 = W_lm each head predicts exactly what the LM head does
    rng = np.random.default_rng(1)
    d, V, K, B = 32, 50, 3, 2
    h = rng.standard_normal((B, d))
    Wlm = rng.standard_normal((V, d))
    W1 = np.zeros((K, d, d))
    W2 = np.stack([Wlm] * K)
    logits, _ = os_.medusa_heads(h, W1, W2, Wlm)
    for k in range(1, K + 1):
        assert np.array_equal(logits[:, k], logits[:, 0])


def test_heads_bruteforce_loops():
    rng = np.random.default_rng(2)
    d, V, K = 5, 7, 2
    h = rng.standard_normal((1, d)); W1 = rng.standard_normal((K, d, d)); W2 = rng.standard_normal((K, V, d))
    Wlm = rng.standard_normal((V, d))
    logits, _ = os_.medusa_heads(h, W1, W2, Wlm)
    for k in range(K):
        a = []
        for i in range(d):
            u = sum(W1[k, i, j] * h[0, j] for j in range(d))
            a.append(u / (1 + math.exp(-u)) + h[0, i])
        for v in range(V):
            assert abs(logits[0, k + 1, v] - sum(W2[k, v, i] * a[i] for i in range(d))) < 1e-12
    for v in range(V):
        assert abs(logits[0, 0, v] - sum(Wlm[v, j] * h[0, j] for j in range(d))) < 1e-12


# ---------------------------------------------------------------- top-k

def _topk_select(row, k):
    taken, out = set(), []
    for _ in range(k):
        best = None
        for i, x in enumerate(row):
            if i in taken:
                continue
            if best is None or x > row[best]:
                best = i
        taken.add(best)
        out.append(best)
    return out


def test_topk_vs_selection_with_ties():
    rng = np.random.default_rng(3)
    for trial in range(50):
        n = int(rng.integers(5, 60))
        row = rng.integers(-4, 4, n).astype(np.float64)       # many exact ties
        k = int(rng.integers(1, n + 1))
        idx, val = os_.topk(row, k)
        assert list(idx) == _topk_select(list(row), k)
        assert np.array_equal(val, row[idx])


def test_tree_expand_tokens_and_positions():
    t = ot.cartesian_tree((3, 2))
    topk_idx = np.array([[[100, 101, 102], [200, 201, 202], [300, 301, 302]]])
    tokens, pos = os_.tree_expand(topk_idx, t, np.array([7]))
    assert tokens[0, 0] == 100
    for i in range(1, t.T):
        assert tokens[0, i] == 100 * (t.depth[i] + 1) + t.paths[i][-1]
        assert pos[0, i] == 7 + len(t.paths[i])


# ---------------------------------------------------------------- rope + attention

def test_rope_hand_values():
    g = json.load(open(os.path.join(GOLDEN, "rope_hand.json")))
    for c in g["cases"]:
        np.testing.assert_allclose(os_.rope(np.array(c["x"]), c["pos"]), np.array(c["out"]), rtol=0, atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p in (0, 5, 1000):
        r = os_.rope(q, p)
        # each (m, m+Dh/2) pair keeps its length
        assert np.allclose(r[:32] ** 2 + r[32:] ** 2, q[:32] ** 2 + q[32:] ** 2)
    # dot products depend only on the position difference
    a = os_.rope(q, 17) @ os_.rope(k, 5)
    b = os_.rope(q, 1017) @ os_.rope(k, 1005)
    assert abs(a - b) < 1e-9


def _causal_path_attention(q, k, v, Kc, Vc, L, tree, i, h, theta):
    """Check (b): node i's root path run as its own sequence with a plain causal mask (torch SDPA)."""
    path = ot.ancestors(tree, i)
    n = L + len(path)
    keys = np.concatenate([Kc[:L, h], np.stack([os_.rope(k[j, h], L + m, theta) for m, j in enumerate(path)])])
    vals = np.concatenate([Vc[:L, h], v[path, h]])
    qs = np.zeros((n, q.shape[-1]))
    qs[L:] = np.stack([os_.rope(q[j, h], L + m, theta) for m, j in enumerate(path)])
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool))
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qs)[None, None], torch.from_numpy(keys)[None, None], torch.from_numpy(vals)[None, None],
        attn_mask=mask)
    return out[0, 0, -1].numpy()


@pytest.mark.parametrize("maker,L", [(lambda: ot.cartesian_tree((3, 2)), 9), (lambda: ot.scored_tree_greedy(3, 4, 20), 17),
                                     (lambda: ot.cartesian_tree((1, 1, 1)), 5), (lambda: ot.cartesian_tree(()), 12)])
def test_tree_attention_equals_per_path_causal_attention(maker, L):
    t = maker()
    rng = np.random.default_rng(5)
    H, Dh, T = 2, 8, t.T
    q, k, v = (rng.standard_normal((1, T, H, Dh)) for _ in range(3))
    Kc, Vc = rng.standard_normal((1, L + 4, H, Dh)), rng.standard_normal((1, L + 4, H, Dh))
    o, k_rot = os_.tree_attention(q, k, v, Kc, Vc, np.array([L]), t, bf16_store=False)
    for i in range(T):
        for h in range(H):
            ref = _causal_path_attention(q[0], k[0], v[0], Kc[0], Vc[0], L, t, i, h, 10000.0)
            np.testing.assert_allclose(o[0, i, h], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(k_rot[0, i], os_.rope(k[0, i], L + t.depth[i]))


def test_tree_attention_paged_equals_contiguous():
    t = ot.cartesian_tree((2, 2))
    rng = np.random.default_rng(6)
    B, H, Dh, ps = 2, 2, 4, 4
    lens = np.array([9, 14])
    cap = 20
    Kc, Vc = rng.standard_normal((B, cap, H, Dh)), rng.standard_normal((B, cap, H, Dh))
    q, k, v = (rng.standard_normal((B, t.T, H, Dh)) for _ in range(3))
    npg = cap // ps
    perm = rng.permutation(B * npg)
    table = perm.reshape(B, npg)
    pool_k, pool_v = np.zeros((B * npg, ps, H, Dh)), np.zeros((B * npg, ps, H, Dh))
    for b in range(B):
        for s in range(cap):
            pool_k[table[b, s // ps], s % ps] = Kc[b, s]
            pool_v[table[b, s // ps], s % ps] = Vc[b, s]
    o1, _ = os_.tree_attention(q, k, v, Kc, Vc, lens, t, bf16_store=False)
    o2, _ = os_.tree_attention(q, k, v, pool_k, pool_v, lens, t, bf16_store=False, page_table=table, page_size=ps)
    assert np.array_equal(o1, o2)


# ---------------------------------------------------------------- verifier statistics

def test_row_stats_vs_scipy():
    rng = np.random.default_rng(7)
    for tau in (0.3, 0.7, 1.0, 2.5):
        z = rng.standard_normal(1000) * 3
        st = os_.row_stats(z, tau)
        assert abs(st["logZ"] - scipy.special.logsumexp(z / tau)) < 1e-10
        p = scipy.special.softmax(z / tau)
        assert abs(st["H"] - scipy.stats.entropy(p)) < 1e-10
        assert st["argmax"] == int(np.argmax(z)) and st["max"] == z.max()


def test_row_stats_closed_forms():
    V = 32000
    st = os_.row_stats(np.full(V, 1.25), 0.7)
    assert abs(st["H"] - math.log(V)) < 1e-9                # uniform: H = ln V
    assert abs(st["logZ"] - (1.25 / 0.7 + math.log(V))) < 1e-9
    assert st["argmax"] == 0                                  # ties: smallest index
    z = np.zeros(10); z[3] = z[7] = 2.0
    st = os_.row_stats(z, 0.0)
    assert st["argmax"] == 3 and st["H"] == 0.0 and st["logZ"] == 0.0
    # a very peaked row has ~zero entropy
    z = np.zeros(100); z[5] = 1000.0
    assert os_.row_stats(z, 1.0)["H"] < 1e-12


def test_edge_logits_pick_parent_row():
    t = ot.cartesian_tree((2, 2))
    B, T, V = 1, t.T, 9
    z = np.arange(B * T * V, dtype=np.float64).reshape(B * T, V)
    tokens = np.array([[0, 1, 2, 3, 4, 5, 6]])
    e = os_.edge_logits(z, tokens, t)
    for c in range(1, T):
        assert e[0, c] == t.parent[c] * V + tokens[0, c]


# ---------------------------------------------------------------- acceptance

def _planted(t, rng, V=20, B=1):
    tokens = rng.integers(0, V, (B, t.T))
    stats = [{"argmax": int(rng.integers(0, V)), "max": 0.0, "logZ": 0.0, "H": 0.0} for _ in range(B * t.T)]
    # plant matches so that some deep paths pass
    for b in range(B):
        for c in range(1, t.T):
            if rng.random() < 0.5:
                stats[b * t.T + t.parent[c]]["argmax"] = int(tokens[b, c])
    return tokens, stats


def _greedy_walk(tokens_b, stats, b, t):
    """'Notes on Medusa' section 3: take the verifier's token at the current node; if a child carries
    it, descend into that child; stop when no child matches."""
    node, path = 0, [0]
    while True:
        want = stats[b * t.T + node]["argmax"]
        kids = [c for c in range(t.T) if t.parent[c] == node and tokens_b[c] == want]
        if not kids:
            return path
        node = kids[0]
        path.append(node)


@pytest.mark.parametrize("maker", [lambda: ot.cartesian_tree((3, 2)), lambda: ot.scored_tree_greedy(4, 5, 40)])
def test_greedy_acceptance_equals_tree_walk(maker):
    t = maker()
    rng = np.random.default_rng(8)
    for trial in range(200):
        tokens, stats = _planted(t, rng)
        # siblings carry distinct tokens (distinct top-k entries of one head)
        for c in range(1, t.T):
            sib = [s for s in range(1, c) if t.parent[s] == t.parent[c]]
            while tokens[0, c] in tokens[0, sib]:
                tokens[0, c] = (tokens[0, c] + 1) % 20
        paths, n = os_.accept_path(stats, np.zeros_like(tokens, dtype=float), tokens, t, "greedy")
        walk = _greedy_walk(tokens[0], stats, 0, t)
        assert paths[0] == walk and n[0] == len(walk)


def test_typical_at_zero_temperature_is_greedy():
    # check (c): summary page, "Typical Acceptance Scheme": at temperature 0 typical acceptance is greedy
    t = ot.scored_tree_greedy(4, 5, 40)
    rng = np.random.default_rng(9)
    for trial in range(100):
        tokens, stats = _planted(t, rng, B=2)
        e = rng.standard_normal(tokens.shape)
        g = os_.accept_path(stats, e, tokens, t, "greedy")
        ty = os_.accept_path(stats, e, tokens, t, "typical", eps=0.09, delta=0.3, tau=0.0)
        assert g == ty


def test_first_token_always_accepted():
    # check (d): the root is accepted even when every verifier row rejects every child
    t = ot.scored_tree_greedy(4, 10, 64)
    T, V = t.T, 1000
    tokens = np.arange(T)[None, :] + 1
    stats = [{"argmax": 0, "max": 50.0, "logZ": 50.0 / 0.7, "H": 0.0} for _ in range(T)]
    e = np.full((1, T), -50.0)
    for mode, tau in (("greedy", 0.0), ("typical", 0.7), ("typical", 0.0)):
        paths, n = os_.accept_path(stats, e, tokens, t, mode, 0.09, 0.3, tau)
        assert paths == [[0]] and n == [1]


def test_uniform_rows_accept_every_child():
    # closed form: uniform verifier rows have H = ln V and p = 1/V > delta/V >= min(eps, delta e^-H)
    t = ot.scored_tree_greedy(4, 10, 64)
    V, tau = 32000, 0.7
    z = np.full(V, 0.5)
    st = os_.row_stats(z, tau)
    stats = [st] * t.T
    tokens = np.arange(t.T)[None, :]
    e = np.full((1, t.T), 0.5)
    paths, n = os_.accept_path(stats, e, tokens, t, "typical", 0.09, 0.3, tau)
    deepest = [i for i in range(t.T) if t.depth[i] == t.max_depth]
    assert n == [t.max_depth + 1] and paths[0][-1] == min(deepest)


def test_typical_bruteforce_over_paths():
    # longest accepted prefix over all branches; equal lengths -> smallest packed index of the end node
    t = ot.cartesian_tree((3, 2, 2))
    rng = np.random.default_rng(10)
    for trial in range(200):
        tokens = rng.integers(0, 50, (1, t.T))
        stats = [{"argmax": 0, "max": 0.0, "logZ": float(rng.uniform(2, 6)), "H": float(rng.uniform(0, 4))}
                 for _ in range(t.T)]
        e = rng.uniform(-2, 6, (1, t.T))
        paths, n = os_.accept_path(stats, e, tokens, t, "typical", 0.09, 0.3, 0.7)
        ok = {}
        for i in range(1, t.T):
            st = stats[t.parent[i]]
            ok[t.paths[i]] = math.exp(e[0, i] / 0.7 - st["logZ"]) > min(0.09, 0.3 * math.exp(-st["H"]))
        best = ()
        for p in sorted(ok, key=lambda p: (-len(p), p)):
            if all(ok[p[:m]] for m in range(1, len(p) + 1)):
                best = p
                break
        assert [t.paths[j] for j in paths[0]] == [best[:m] for m in range(len(best) + 1)]


# ---------------------------------------------------------------- compaction

def test_kv_compact_equals_recompute():
    # check (e): the accepted rows re-rotated as a plain sequence at L..L+n-1, appended to the prefix
    t = ot.scored_tree_greedy(3, 4, 20)
    rng = np.random.default_rng(11)
    B, H, Dh, L = 2, 2, 8, 6
    lens = np.array([L, L + 3])
    q, k, v = (rng.standard_normal((B, t.T, H, Dh)) for _ in range(3))
    Kc, Vc = rng.standard_normal((B, 16, H, Dh)), rng.standard_normal((B, 16, H, Dh))
    _, k_rot = os_.tree_attention(q, k, v, Kc, Vc, lens, t, bf16_store=False)
    paths = [ot.ancestors(t, 17), ot.ancestors(t, 4)]
    Kn, Vn, new_len = os_.kv_compact(Kc, Vc, k_rot, v, paths, lens)
    for b in range(B):
        Lb = int(lens[b])
        assert new_len[b] == Lb + len(paths[b])
        seq_k = np.stack([os_.rope(k[b, node], Lb + j) for j, node in enumerate(paths[b])])
        assert np.array_equal(Kn[b, Lb:Lb + len(paths[b])], seq_k)
        assert np.array_equal(Vn[b, Lb:Lb + len(paths[b])], v[b, paths[b]])
        assert np.array_equal(Kn[b, :Lb], Kc[b, :Lb]) and np.array_equal(Kn[b, Lb + len(paths[b]):], Kc[b, Lb + len(paths[b]):])


# ---------------------------------------------------------------- margins

def test_margins():
    logits = np.array([[[5.0, 3.0, 4.9995, 1.0]]])
    assert abs(om.head_margin(logits, 1) - 0.0005) < 1e-12
    assert abs(om.head_margin(logits, 3) - 0.0005) < 1e-12
    z = np.array([[1.0, 2.0, 3.0], [1.0, 1.0005, 0.0]])
    assert om.unique_argmax_rows(z) == [0]
