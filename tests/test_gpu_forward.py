"""GPU parity of the full verify forward and of its layer calls against the oracle.

Layer calls (embed, rmsnorm, linear in its three forms, the split product and its
closing add_rmsnorm): each output element within one bf16 unit of the float64 oracle
plus the fp32 arithmetic's own error bound (both round once; they can differ only
where the two sums straddle a rounding boundary), at shapes with ragged tails.

The forward (two layers: the 7B mini and full 7B width): tree tokens, path, n_acc
and new lengths bit-exact (every decision's oracle margin is checked to exceed twice
the logit difference that the final rows' difference induces);
residual stream, final rows, every layer's rotated keys and values per row within
2e-2 of the oracle; the verifier argmax on every row whose top-2 gap exceeds twice
that difference, and logZ within it; the compacted caches equal the GPU's own
keys/values at the path rows, bit for bit, with every other row untouched.
"""

import functools

import numpy as np
import pytest
import torch

from oracle import forward as ofw
from oracle import margins as om
from oracle import step as ostep
from oracle import tree as otree
from tests.parity_util import REL_TOL, SEEDS, note, rel_err_rows
from workloads import make_inputs
from workloads.configs import FORWARD_CASES
from workloads.gen import forward_inputs, layer_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _dev(a):
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def _rand_bf16(rng, shape, std=1.0):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return ostep.round_bf16(x.astype(np.float64))


def _to_bits(x64):
    """float64 values that are bf16 numbers -> bf16 patterns."""
    return (x64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _ulp(ref):
    """One bf16 unit in the last place of each reference value (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
    return np.exp2(e - 7)


def _bad(g_bits, ref, fp32_err=0.0):
    """Elements further from the float64 result than one bf16 unit plus the fp32
    arithmetic's own error bound ``fp32_err`` (both sides round once; they can differ
    by a unit only where the two sums straddle a rounding boundary)."""
    g = ostep.to_f64(g_bits)
    return int((np.abs(g - ref) > _ulp(ref) * 1.0001 + fp32_err + 1e-30).sum())


def _dot_err(x, W, K):
    """Bound on the fp32 error of the K-term dot products x W^T in any summation order:
    gamma_K * sum |x||w| with gamma_K ~ K * 2^-24 (taken twice for margin)."""
    return K * 2.0 ** -23 * (np.abs(x) @ np.abs(W).T)


# On 256 CUs the tile width follows N and the row blocks: 48 columns (the small shapes),
# 96 (22000; 6000 over three row blocks), 128 (31992) or the 4-wave 64 x 64 tile (40000),
# each with a ragged last tile.
LIN_SHAPES = [(64, 192, 256), (37, 200, 320), (130, 96, 1376), (64, 512, 4096), (64, 22000, 256),
              (130, 6000, 288), (40, 31992, 256), (64, 40000, 256)]


@pytest.mark.parametrize("M,N,K", LIN_SHAPES)
def test_linear_plain_and_residual(M, N, K):
    import medusa_tree_verification_heads_amd as mdt
    note(f"linear M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 1000 + N + K)
    x = _rand_bf16(rng, (M, K))
    W = _rand_bf16(rng, (N, K), K ** -0.5)
    r = _rand_bf16(rng, (M, N))
    xd, Wd, rd = _dev(_to_bits(x)), _dev(_to_bits(W)), _dev(_to_bits(r))
    y = mdt.linear(xd, Wd)
    bound = _dot_err(x, W, K)
    assert _bad(_bits(y), ofw.linear(x, _to_bits(W)), bound) == 0
    # in place on the residual
    mdt.linear(xd, Wd, residual=rd, out=rd)
    assert _bad(_bits(rd), ofw.linear(x, _to_bits(W), r), bound) == 0


@pytest.mark.parametrize("M,N,K,nsplit", [(64, 512, 4096, 8), (37, 200, 1376, 2), (130, 96, 1024, 3),
                                          (64, 4096, 11008, 8), (16, 6656, 1536, 12), (5, 12288, 512, 4)])
def test_linear_split_and_add_rmsnorm(M, N, K, nsplit):
    """The slices' fp32 products add up to the product (each within the fp32 dot-product
    bound), and add_rmsnorm closes them into the residual and normalises the new row."""
    import medusa_tree_verification_heads_amd as mdt
    note(f"linear_split M={M} N={N} K={K} nsplit={nsplit}")
    rng = np.random.default_rng(N + K + nsplit)
    x = _rand_bf16(rng, (M, K))
    W = _rand_bf16(rng, (N, K), K ** -0.5)
    r = _rand_bf16(rng, (M, N))
    g = ostep.round_bf16(1 + 0.1 * rng.standard_normal(N))
    part = mdt.linear_split(_dev(_to_bits(x)), _dev(_to_bits(W)), nsplit)
    ks = -(-(-(-K // nsplit)) // 32) * 32
    bound = _dot_err(x, W, K)
    p = part.cpu().numpy().astype(np.float64)
    for s_ in range(nsplit):
        sl = slice(s_ * ks, min(K, (s_ + 1) * ks))
        assert np.all(np.abs(p[s_] - x[:, sl] @ W[:, sl].T) <= bound + 1e-30)
    xr = _dev(_to_bits(r))
    h = mdt.add_rmsnorm(part, xr, _dev(_to_bits(g)), 1e-6)
    x_new = ofw.linear(x, _to_bits(W), r)
    assert _bad(_bits(xr), x_new, bound) == 0
    # the norm is of the row as stored: where an element of x was rounded one unit apart
    # from the oracle's, the normalised element moves by that difference times r * g
    ref_h = ofw.rmsnorm(x_new, g, 1e-6)
    dx = np.abs(ostep.to_f64(_bits(xr)) - x_new)
    rr = 1.0 / np.sqrt(np.mean(x_new * x_new, axis=1, keepdims=True) + 1e-6)
    assert _bad(_bits(h), ref_h, (N + 8) * 2.0 ** -24 * np.abs(ref_h) + 1.01 * dx * rr * np.abs(g)) == 0


@pytest.mark.parametrize("M,N,K", [(64, 3 * 192, 256), (37, 3 * 512, 512)])
def test_linear_segments(M, N, K):
    import medusa_tree_verification_heads_amd as mdt
    rng = np.random.default_rng(7 + M)
    x = _rand_bf16(rng, (M, K))
    W = _rand_bf16(rng, (N, K), K ** -0.5)
    y = mdt.linear(_dev(_to_bits(x)), _dev(_to_bits(W)), nseg=3)
    assert y.shape == (3, M, N // 3)
    ref = ofw.linear(x, _to_bits(W))
    bound = _dot_err(x, W, K)
    for q in range(3):
        cols = slice(q * (N // 3), (q + 1) * (N // 3))
        assert _bad(_bits(y[q]), ref[:, cols], bound[:, cols]) == 0


@pytest.mark.parametrize("M,F,K", [(64, 1376, 512), (37, 48, 256), (64, 11008 // 4, 4096), (64, 11008, 256),
                                   (50, 16000, 256), (64, 20000, 256)])
def test_linear_swiglu(M, F, K):
    import medusa_tree_verification_heads_amd as mdt
    note(f"swiglu M={M} F={F} K={K}")
    rng = np.random.default_rng(F + K + M)
    h = _rand_bf16(rng, (M, K))
    Wg = _rand_bf16(rng, (F, K), K ** -0.5)
    Wu = _rand_bf16(rng, (F, K), K ** -0.5)
    W = mdt.interleave_gate_up(_dev(_to_bits(Wg)), _dev(_to_bits(Wu)))
    a = mdt.linear(_dev(_to_bits(h)), W, act=mdt.ACT_SWIGLU)
    zg, zu = h @ Wg.T, h @ Wu.T
    ref = ostep.round_bf16(ofw.swiglu(zg, zu))
    # first-order propagation of the dot-product bounds through silu(g) * u
    # (|d silu/dg| <= 1.1), plus the exponential's few-ulp fp32 error
    eg, eu = _dot_err(h, Wg, K), _dot_err(h, Wu, K)
    bound = 1.1 * eg * np.abs(zu) + np.abs(ofw.swiglu(zg, np.ones_like(zg))) * eu + 1e-6 * np.abs(ref)
    assert _bad(_bits(a), ref, bound) == 0


@pytest.mark.parametrize("M,d", [(64, 512), (13, 4096), (1, 136), (5, 6656), (3, 12288), (2, 40968)])
def test_rmsnorm_and_embed(M, d):
    import medusa_tree_verification_heads_amd as mdt
    rng = np.random.default_rng(M + d)
    x = _rand_bf16(rng, (M, d), 3.0)
    g = ostep.round_bf16(1 + 0.1 * rng.standard_normal(d))
    y = mdt.rmsnorm(_dev(_to_bits(x)), _dev(_to_bits(g)), 1e-6)
    ref = ofw.rmsnorm(x, g, 1e-6)
    # fp32 sum of squares (d terms) and the reciprocal square root's couple of ulps
    assert _bad(_bits(y), ref, (d + 8) * 2.0 ** -24 * np.abs(ref)) == 0
    V = 301
    E = _rand_bf16(rng, (V, d))
    tok = rng.integers(-3, V + 3, M).astype(np.int32)
    e = mdt.embed(torch.from_numpy(tok).cuda(), _dev(_to_bits(E)))
    want = np.where(((tok >= 0) & (tok < V))[:, None], E[np.clip(tok, 0, V - 1)], 0.0)
    assert np.array_equal(ostep.to_f64(_bits(e)), want)


def _seed(dw):
    """A forward case's own seed (oracle/find_seeds.py --forward), else its step case's."""
    for key in (f"fwd:{dw.name}", dw.base.name):
        if key in SEEDS:
            return SEEDS[key]["seed"]
    return 1


@functools.lru_cache(maxsize=None)
def _inputs(name):
    dw = FORWARD_CASES[name]
    seed = _seed(dw)
    inp = make_inputs(dw.base, seed, parts=("h", "W1", "W2", "Wlm"))
    return dw, inp, forward_inputs(dw, seed), [layer_inputs(dw, seed, l) for l in range(dw.n_layers)]


@functools.lru_cache(maxsize=None)
def _oracle(name, run_idx):
    dw, inp, fin, layers = _inputs(name)
    run = dw.base.accept[run_idx]
    note(f"oracle forward {name} {run}")
    return ofw.forward(dw, inp, fin, layers, otree.build_tree(dw.base), run.mode, run.temperature, run.eps,
                       run.delta)


def _gpu(name, run_idx):
    from medusa_tree_verification_heads_amd.forward import VerifyForward
    dw, inp, fin, layers = _inputs(name)
    run = dw.base.accept[run_idx]
    note(f"gpu forward {name} {run}")
    f = VerifyForward.from_numpy(dw, inp, fin, layers, mode=run.mode, temperature=run.temperature, eps=run.eps,
                                 delta=run.delta)
    f.run()
    return f.outputs()


FWD_RUNS = [(n, i) for n in FORWARD_CASES for i in range(len(FORWARD_CASES[n].base.accept))]


@pytest.mark.parametrize("name,run_idx", FWD_RUNS)
def test_forward(name, run_idx):
    dw, inp, fin, layers = _inputs(name)
    w = dw.base
    run = w.accept[run_idx]
    tree = otree.build_tree(w)
    ref = _oracle(name, run_idx)
    hm = om.head_margin(ref["logits"], w.k_cfg)
    note(f"{name} run {run_idx}: head margin {hm:.3g}, n_acc {ref['n_acc']}")
    assert hm >= 1e-3
    g = _gpu(name, run_idx)
    assert np.array_equal(g["tokens"], ref["tokens"])
    err_x = rel_err_rows(ostep.to_f64(g["x_last"]), ref["x_last"])
    err_f = rel_err_rows(ostep.to_f64(g["xf"]), ref["xf"])
    note(f"{name}: residual stream rel err {err_x:.2e}, final rows {err_f:.2e}")
    assert err_x <= REL_TOL and err_f <= REL_TOL
    for l in range(dw.n_layers):
        ek = rel_err_rows(ostep.to_f64(g["k_rot"][l]), ref["k_rot"][l])
        ev = rel_err_rows(ostep.to_f64(g["v"][l]).reshape(ref["v"][l].shape), ref["v"][l])
        note(f"{name}: layer {l} k_rot rel err {ek:.2e}, v {ev:.2e}")
        assert ek <= REL_TOL and ev <= REL_TOL
    # The final rows already differ from the oracle's by up to REL_TOL; the logits of a row
    # then differ by dz = W_lm (xf_gpu - xf_oracle) plus the GPU product's own fp32 error
    # (~1e-6 relative).  Every decision whose oracle margin exceeds twice max |dz| of the
    # rows involved is compared.
    dxf = ostep.to_f64(g["xf"]) - ref["xf"]
    zb = np.abs(dxf @ ostep.to_f64(inp["Wlm"]).T).max(axis=1) + 1e-5 * np.abs(ref["z"]).max()
    tau = run.temperature or 1.0
    em = om.edge_margins(ref["z"], ref["stats"], ref["tokens"], tree, run.mode, run.eps, run.delta,
                         run.temperature)
    par = np.array([tree.parent[c] if c else 0 for c in range(tree.T)])
    edge_bound = np.stack([2 * zb[b * tree.T + par] / tau for b in range(w.B)])
    note(f"{name}: logit error bound max {zb.max():.3g}; edge margin min {em.min():.3g}")
    assert (em > edge_bound).all()
    st = np.ascontiguousarray(g["stats"]).view(np.dtype([("max", np.float32), ("argmax", np.int32),
                                                          ("logZ", np.float32), ("entropy", np.float32)]))
    st = st.reshape(-1)
    z = ref["z"]
    clear = [r for r in range(z.shape[0]) if np.diff(np.partition(z[r], -2)[-2:])[0] > 2 * zb[r]]
    note(f"{name}: {len(clear)} of {z.shape[0]} rows with a clear argmax")
    assert len(clear) >= z.shape[0] // 2
    assert all(int(st["argmax"][r]) == ref["stats"][r]["argmax"] for r in clear)
    if run.temperature > 0:
        lz = np.array([s["logZ"] for s in ref["stats"]])
        assert (np.abs(st["logZ"] - lz) <= zb / run.temperature + 1e-5 * np.abs(lz)).all()
    assert g["n_acc"].tolist() == ref["n_acc"]
    for b in range(w.B):
        n = ref["n_acc"][b]
        assert g["path"][b, :n].tolist() == ref["paths"][b]
        assert (g["path"][b, n:] == -1).all()
    assert g["new_len"].tolist() == ref["new_len"]
    # compaction: path rows are the GPU's own keys/values, the rest untouched
    for l in range(dw.n_layers):
        K0, V0 = layers[l]["Kc"], layers[l]["Vc"]
        Kg, Vg = g["Kc"][l], g["Vc"][l]
        vg = g["v"][l].reshape(w.B, tree.T, w.H, w.Dh)
        for b in range(w.B):
            L = int(inp["prefix_len"][b])
            n = ref["n_acc"][b]
            for j, node in enumerate(ref["paths"][b]):
                assert np.array_equal(Kg[b, L + j], g["k_rot"][l][b, node])
                assert np.array_equal(Vg[b, L + j], vg[b, node])
            keep = np.ones(Kg.shape[1], dtype=bool)
            keep[L:L + n] = False
            assert np.array_equal(Kg[b, keep], K0[b, keep]) and np.array_equal(Vg[b, keep], V0[b, keep])


def test_compact_layers_planted_paths():
    """Deep paths (the forward's own paths are short on random weights): layer l's rows
    of a planted path land at prefix_len + j in layer l's cache, nothing else moves."""
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.forward import VerifyForward
    dw, inp, fin, layers = _inputs("7b-mini-x2")
    w = dw.base
    f = VerifyForward.from_numpy(dw, inp, fin, layers)
    f.run()
    torch.cuda.synchronize()
    tree = otree.build_tree(w)
    deepest = max(range(tree.T), key=lambda i: (tree.depth[i], -i))
    path = otree.ancestors(tree, deepest)
    K0, V0 = f.Kc.clone(), f.Vc.clone()
    p = torch.full((w.B, f.path.shape[1]), -1, dtype=torch.int32, device="cuda")
    p[0, :len(path)] = torch.tensor(path, dtype=torch.int32)
    n = torch.tensor([len(path)], dtype=torch.int32, device="cuda")
    lens = f.prefix_len.clone()
    new_len = torch.empty_like(lens)
    B, T, H, Dh = w.B, tree.T, w.H, w.Dh
    v = f.qkv[:, 2].view(dw.n_layers, B, T, H, Dh)
    mdt.kv_compact_layers(p, n, f.k_rot, v, f.caches[0], lens, f.Kc.stride(0), new_prefix_len=new_len)
    torch.cuda.synchronize()
    L = int(lens[0])
    assert int(new_len[0]) == L + len(path)
    for l in range(dw.n_layers):
        for j, node in enumerate(path):
            assert torch.equal(f.Kc[l, 0, L + j].view(torch.int16), f.k_rot[l, 0, node].view(torch.int16))
            assert torch.equal(f.Vc[l, 0, L + j].view(torch.int16), v[l, 0, node].view(torch.int16))
        keep = torch.ones(f.Kc.shape[2], dtype=torch.bool, device="cuda")
        keep[L:L + len(path)] = False
        assert torch.equal(f.Kc[l, 0, keep].view(torch.int16), K0[l, 0, keep].view(torch.int16))
        assert torch.equal(f.Vc[l, 0, keep].view(torch.int16), V0[l, 0, keep].view(torch.int16))


def test_forward_graph_replay_matches_eager():
    """The whole forward captured as one HIP graph gives the eager outputs on every replay,
    with eager runs in between (compaction rewrites the same rows: the prefix length
    input is not advanced)."""
    from medusa_tree_verification_heads_amd.forward import VerifyForward
    dw, inp, fin, layers = _inputs("7b-mini-x2")
    f = VerifyForward.from_numpy(dw, inp, fin, layers, mode="typical", temperature=0.7)
    f.run()
    eager = f.outputs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        f.run()

    def same(a, b):
        for k in a:
            assert np.array_equal(a[k], b[k]), k

    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        same(eager, f.outputs())
        f.run()
        torch.cuda.synchronize()
        same(eager, f.outputs())



@pytest.mark.parametrize("M,N,K", [(1, 8, 32), (1, 96, 64), (17, 40, 96), (65, 8, 32)])
def test_linear_smallest_shapes(M, N, K):
    """Single rows, a single 8-column group, a single 32-wide k-step, a second row tile."""
    import medusa_tree_verification_heads_amd as mdt
    rng = np.random.default_rng(M * 7 + N + K)
    x = _rand_bf16(rng, (M, K))
    W = _rand_bf16(rng, (N, K), K ** -0.5)
    r = _rand_bf16(rng, (M, N))
    xd, Wd, rd = _dev(_to_bits(x)), _dev(_to_bits(W)), _dev(_to_bits(r))
    bound = _dot_err(x, W, K)
    assert _bad(_bits(mdt.linear(xd, Wd)), ofw.linear(x, _to_bits(W)), bound) == 0
    mdt.linear(xd, Wd, residual=rd, out=rd)
    assert _bad(_bits(rd), ofw.linear(x, _to_bits(W), r), bound) == 0
    if N % 32 == 0:
        F = N // 2
        Wg, Wu = W[0::2][:F], W[1::2][:F]
        a = mdt.linear(xd, mdt.interleave_gate_up(_dev(_to_bits(Wg)), _dev(_to_bits(Wu))), act=mdt.ACT_SWIGLU)
        zg, zu = x @ Wg.T, x @ Wu.T
        ref = ostep.round_bf16(ofw.swiglu(zg, zu))
        b2 = 1.1 * _dot_err(x, Wg, K) * np.abs(zu) + np.abs(ofw.swiglu(zg, np.ones_like(zg))) * _dot_err(x, Wu, K)
        assert _bad(_bits(a), ref, b2 + 1e-6 * np.abs(ref)) == 0
    if K >= 64:
        part = mdt.linear_split(xd, Wd, 2)
        assert np.allclose(part.sum(0).cpu().numpy(), x @ W.T, rtol=0, atol=float(bound.max()) * 2 + 1e-6)


def test_compact_layers_paged():
    """Layered compaction into a paged pool: layer l's pool sits cache_layer_stride
    elements after layer 0's; the page table is shared."""
    import medusa_tree_verification_heads_amd as mdt
    B, T, H, Dh, nL, page, npages = 2, 10, 2, 128, 3, 16, 12
    rng = np.random.default_rng(5)
    k_rot = torch.from_numpy(rng.standard_normal((nL, B, T, H, Dh)).astype(np.float32)).to(torch.bfloat16).cuda()
    v = torch.from_numpy(rng.standard_normal((nL, B, T, H, Dh)).astype(np.float32)).to(torch.bfloat16).cuda()
    Kp = torch.zeros((nL, npages, page, H, Dh), dtype=torch.bfloat16, device="cuda")
    Vp = torch.zeros_like(Kp)
    table = torch.tensor([[3, 7, 1, -1], [0, 9, 4, 11]], dtype=torch.int32, device="cuda")
    cache = mdt.KVCache(Kp[0], Vp[0], table, page)
    lens = torch.tensor([14, 30], dtype=torch.int32, device="cuda")
    path = torch.tensor([[0, 2, 7, -1], [0, 1, -1, -1]], dtype=torch.int32, device="cuda")
    n = torch.tensor([3, 2], dtype=torch.int32, device="cuda")
    new_len = mdt.kv_compact_layers(path, n, k_rot, v, cache, lens, Kp.stride(0))
    torch.cuda.synchronize()
    assert new_len.cpu().tolist() == [17, 32]
    tb = table.cpu().numpy()
    for l in range(nL):
        for b, L in enumerate([14, 30]):
            for j, node in enumerate(path[b, :int(n[b])].cpu().tolist()):
                slot = L + j
                pg, off = tb[b, slot // page], slot % page
                assert torch.equal(Kp[l, pg, off].view(torch.int16), k_rot[l, b, node].view(torch.int16))
                assert torch.equal(Vp[l, pg, off].view(torch.int16), v[l, b, node].view(torch.int16))
    written = sum(int(n[b]) for b in range(B)) * nL
    assert int((Kp.view(torch.int16) != 0).any(dim=-1).any(dim=-1).sum()) == written


@pytest.mark.parametrize("reuse", [True, False])
@pytest.mark.parametrize("name", ["7b-mini-x2", "7b-mini-B2-x2"])
def test_forward_loop(name, reuse):
    """Three chained steps through both layers: each step starts from the final normed row
    of the last accepted node, the new prefix length and the compacted caches.  The GPU
    chain is compared with the oracle chain (both from the drawn inputs) while the two
    agree: head logits and final rows within 2e-2, top-k rows exactly where the oracle's
    gaps exceed twice the observed logit difference, accepted paths exactly where every
    edge margin exceeds the bound that the final rows' difference puts on the logits.
    Every step is also checked by properties of the GPU's own values (its top-k, tree
    tokens, path structure, carried row, new lengths), and the prefix rows of every
    layer's cache stay untouched."""
    from medusa_tree_verification_heads_amd.forward import ForwardLoop, VerifyForward
    from tests.parity_util import clear_topk_rows, exact_topk
    S = 3
    dw = FORWARD_CASES[name]
    w = dw.base
    seed = SEEDS[f"fwd:{name}@loop{S}"]["seed"]
    inp = make_inputs(w, seed, parts=("h", "W1", "W2", "Wlm"), steps=S)
    fin = forward_inputs(dw, seed)
    layers = [layer_inputs(dw, seed, l, steps=S) for l in range(dw.n_layers)]
    tree = otree.build_tree(w)
    T, B = tree.T, w.B
    Wlm = ostep.to_f64(inp["Wlm"])
    for run in w.accept:
        ref = ofw.forward_loop(dw, inp, fin, layers, tree, S, run.mode, run.temperature, run.eps, run.delta)
        f = VerifyForward.from_numpy(dw, inp, fin, layers, mode=run.mode, temperature=run.temperature, eps=run.eps,
                                     delta=run.delta)
        loop = ForwardLoop(f, S, reuse_lm_head=reuse)
        together, steps_compared = True, 0
        for s in range(S):
            L = loop.lens[s].cpu().numpy()
            loop.run_step(s)
            torch.cuda.synchronize()
            logits = f.logits.cpu().numpy()
            topk = f.topk_idx.cpu().numpy()
            tokens = loop.tokens[s].cpu().numpy()
            n_acc = loop.n_acc[s].cpu().numpy()
            paths = loop.paths[s].cpu().numpy()
            xf_bits = _bits(f.xf)
            for b in range(B):
                for k in range(w.K + 1):
                    assert topk[b, k].tolist() == exact_topk(logits[b, k], w.k_cfg).tolist(), (s, b, k)
                for i in range(T):
                    assert tokens[b, i] == topk[b, tree.depth[i], tree.rank[i]], (s, b, i)
                path = paths[b, :n_acc[b]].tolist()
                assert path[0] == 0 and all(tree.parent[path[j]] == path[j - 1] for j in range(1, len(path)))
                assert np.array_equal(_bits(loop.h[s + 1])[b], xf_bits[b * T + path[-1]]), (s, b)
            assert np.array_equal(loop.lens[s + 1].cpu().numpy(), L + n_acc), s
            if not together:
                continue
            r = ref[s]
            assert rel_err_rows(logits.astype(np.float64), r["logits"]) <= REL_TOL, s
            diff = np.abs(logits.astype(np.float64) - r["logits"]).max(axis=-1)
            clear = clear_topk_rows(r["logits"], diff, w.k_cfg)
            for b in range(B):
                for k in range(w.K + 1):
                    if clear[b, k]:
                        assert topk[b, k].tolist() == r["topk_idx"][b, k].tolist(), (s, b, k)
            steps_compared += 1
            if not np.array_equal(tokens, r["tokens"]):
                # a near-tie in the heads (not clear above) gave other candidates: the chains part
                note(f"forward loop {name} {run.mode} step {s}: candidates differ at a near-tie; chains part")
                together = False
                continue
            xf = ostep.to_f64(xf_bits)
            assert rel_err_rows(xf, r["xf"]) <= REL_TOL, s
            em = om.edge_margins(r["z"], r["stats"], r["tokens"], tree, run.mode, run.eps, run.delta,
                                 run.temperature)
            dz = np.abs((xf - r["xf"]) @ Wlm.T).reshape(B, -1).max(axis=1)
            for b in range(B):
                need = max(om.MIN_MARGIN, 4 * dz[b] / (run.temperature or 0.5))
                if np.array_equal(tokens[b], r["tokens"][b]) and em[b].min() >= need:
                    assert paths[b, :n_acc[b]].tolist() == r["paths"][b], (s, b)
            together = n_acc.tolist() == r["n_acc"] and all(
                paths[b, :n_acc[b]].tolist() == r["paths"][b] for b in range(B))
            note(f"forward loop {name} {run.mode} step {s}: {int(clear.sum())}/{clear.size} clear top-k rows, "
                 f"chains agree: {together}")
        assert steps_compared >= 1
        for l in range(dw.n_layers):
            for b in range(B):
                L0 = int(inp["prefix_len"][b])
                assert np.array_equal(_bits(f.Kc[l])[b, :L0], layers[l]["Kc"][b, :L0])
                assert np.array_equal(_bits(f.Vc[l])[b, :L0], layers[l]["Vc"][b, :L0])
