"""Tree attention on the degenerate shapes, bf16 (matrix-core kernel) and fp32 paths.

Summary page, "Tree Attention" step 3: every node attends to the prefix and to its
own ancestors.  A root-only tree is plain decode attention; a chain tree (one
candidate per head) is causal attention over the chain; an empty prefix leaves only
the tree's own keys.  Prefix lengths on and off the 64-key tile boundary, in one batch.
Outputs and rotated keys are compared per row with the oracle within 2e-2.
"""

import numpy as np
import pytest
import torch

from oracle import step as ostep
from oracle import tree as otree
from tests.parity_util import REL_TOL, note, rel_err_rows
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

# name -> cartesian ranks per depth
SHAPES = {"root-only": (), "chain-4": (1, 1, 1, 1), "chain-1": (1,), "cart-3x2": (3, 2), "cart-4x3x2": (4, 3, 2)}
PREFIXES = [0, 1, 63, 64, 65, 128, 300, 0]


def _draw(rng, shape, std, bf16):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return f32_to_bf16_bits(x) if bf16 else x


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_attention_degenerate(shape, dtype, paged):
    import medusa_tree_verification_heads_amd as mdt
    s = SHAPES[shape]
    bf16 = dtype == "bf16"
    H, Dh = (3, 128) if bf16 else (4, 16)
    d = H * Dh
    std = d ** -0.25
    ot = otree.cartesian_tree(s)
    T = ot.T
    B = len(PREFIXES)
    L = np.array(PREFIXES, dtype=np.int32)
    note(f"attention edge {shape} T={T} {dtype} paged={paged} prefixes={PREFIXES}")
    rng = np.random.default_rng(T * 7 + bf16 * 3 + paged)
    q, k, v = (_draw(rng, (B, T, H, Dh), std, bf16) for _ in range(3))
    page = 16
    if paged:
        npg = [max(1, -(-int(L[b]) // page)) for b in range(B)]
        pool = sum(npg) + 2
        perm = rng.permutation(pool)
        pt = np.full((B, max(npg)), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            pt[b, :npg[b]] = perm[o:o + npg[b]]
            o += npg[b]
        Kc, Vc = _draw(rng, (pool, page, H, Dh), std, bf16), _draw(rng, (pool, page, H, Dh), std, bf16)
    else:
        pt = None
        cap = int(L.max()) + 3
        Kc, Vc = _draw(rng, (B, cap, H, Dh), std, bf16), _draw(rng, (B, cap, H, Dh), std, bf16)
    tree = mdt.Tree.cartesian(s)
    assert tree.parent.tolist() == list(ot.parent)
    cache = mdt.KVCache(_dev(Kc), _dev(Vc), None if pt is None else torch.from_numpy(pt).cuda(), page)
    out, k_rot = mdt.tree_attention(_dev(q), _dev(k), _dev(v), cache, torch.from_numpy(L).cuda(),
                                    tree.to_device("cuda"))
    torch.cuda.synchronize()
    ro, rk = ostep.tree_attention(q, k, v, Kc, Vc, L, ot, 10000.0, bf16_store=bf16, page_table=pt, page_size=page)
    go, gk = ostep.to_f64(_host(out)), ostep.to_f64(_host(k_rot))
    eo, ek = rel_err_rows(go, ro), rel_err_rows(gk, rk)
    note(f"  o rel err {eo:.2e}, k_rot rel err {ek:.2e}")
    assert eo <= REL_TOL and ek <= REL_TOL
    # an empty prefix under a root-only tree: the root attends to itself only, so o = v
    if T == 1:
        for b in np.nonzero(L == 0)[0]:
            assert rel_err_rows(go[b], ostep.to_f64(v)[b]) <= (1e-6 if not bf16 else 1e-2)


def test_chain_equals_causal_attention():
    """A chain tree over an empty prefix is causal self-attention over the chain: the last
    node's output from the GPU equals plain causal attention computed here on the rotated
    keys the GPU returned (so only the mask and softmax are under test)."""
    import medusa_tree_verification_heads_amd as mdt
    H, Dh, T = 2, 128, 6
    rng = np.random.default_rng(5)
    q, k, v = (_draw(rng, (1, T, H, Dh), 0.3, True) for _ in range(3))
    Kc = _draw(rng, (1, 4, H, Dh), 0.3, True)
    tree = mdt.Tree.cartesian((1,) * (T - 1))
    L = torch.zeros(1, dtype=torch.int32).cuda()
    out, k_rot = mdt.tree_attention(_dev(q), _dev(k), _dev(v), mdt.KVCache(_dev(Kc), _dev(Kc.copy())), L,
                                    tree.to_device("cuda"))
    torch.cuda.synchronize()
    kr = ostep.to_f64(_host(k_rot))[0]
    vf = ostep.to_f64(v)[0]
    go = ostep.to_f64(_host(out))[0]
    for i in range(T):
        qi = np.stack([ostep.rope(ostep.to_f64(q)[0, i, h], i) for h in range(H)])
        for h in range(H):
            sc = kr[:i + 1, h] @ qi[h] / np.sqrt(Dh)
            p = np.exp(sc - sc.max())
            ref = (p / p.sum()) @ vf[:i + 1, h]
            assert np.max(np.abs(go[i, h] - ref)) <= REL_TOL * np.max(np.abs(ref)), (i, h)


# (cartesian ranks, paged, page size): 106 nodes on 8 waves, 213 nodes on 8 waves of two query
# tiles; page sizes that are not powers of two take the division path of the page lookup
SCHEDULES = {
    "T106-paged24": ((5, 4, 4), True, 24),
    "T213-paged16": ((4, 4, 3, 3), True, 16),
    "T213-contig": ((4, 4, 3, 3), False, 0),
    "T41-paged48": ((4, 3, 2), True, 48),
}


@pytest.mark.parametrize("name", list(SCHEDULES))
def test_attention_key_ranges(name):
    """Few (sequence, head) pairs and long prefixes of mixed length: many key ranges per
    pair, ranges past a short prefix (empty partial states), a partial last tile, the tree
    workgroup, and the paged lookups -- against the oracle, row by row."""
    import medusa_tree_verification_heads_amd as mdt
    s, paged, page = SCHEDULES[name]
    H, Dh = 2, 128
    ot = otree.cartesian_tree(s)
    T = ot.T
    L = np.array([0, 700, 1301], dtype=np.int32)
    B = len(L)
    note(f"attention key ranges {name}: T={T} B={B} prefixes={L.tolist()} paged={paged} page={page}")
    rng = np.random.default_rng(T + 17 * page)
    q, k, v = (_draw(rng, (B, T, H, Dh), 0.3, True) for _ in range(3))
    if paged:
        npg = [max(1, -(-int(L[b]) // page)) for b in range(B)]
        pool = sum(npg) + 3
        perm = rng.permutation(pool)
        pt = np.full((B, max(npg) + 2), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            pt[b, :npg[b]] = perm[o:o + npg[b]]
            o += npg[b]
        Kc, Vc = _draw(rng, (pool, page, H, Dh), 0.3, True), _draw(rng, (pool, page, H, Dh), 0.3, True)
    else:
        pt = None
        Kc, Vc = _draw(rng, (B, int(L.max()) + 5, H, Dh), 0.3, True), _draw(rng, (B, int(L.max()) + 5, H, Dh), 0.3, True)
    tree = mdt.Tree.cartesian(s)
    cache = mdt.KVCache(_dev(Kc), _dev(Vc), None if pt is None else torch.from_numpy(pt).cuda(), page or 16)
    out, k_rot = mdt.tree_attention(_dev(q), _dev(k), _dev(v), cache, torch.from_numpy(L).cuda(),
                                    tree.to_device("cuda"))
    torch.cuda.synchronize()
    ro, rk = ostep.tree_attention(q, k, v, Kc, Vc, L, ot, 10000.0, bf16_store=True, page_table=pt,
                                  page_size=page or 16)
    go, gk = ostep.to_f64(_host(out)), ostep.to_f64(_host(k_rot))
    eo, ek = rel_err_rows(go, ro), rel_err_rows(gk, rk)
    note(f"  o rel err {eo:.2e}, k_rot rel err {ek:.2e}")
    assert eo <= REL_TOL and ek <= REL_TOL


# Per 64-key tile of the prefix: the key's value c in the slowest rotary pair's first
# dimension (rotated by at most ~0.13 rad at these positions), against a query component of
# +30 there, puts the tile's scores near -30 c / sqrt(Dh): rising tiles move a row's maximum
# up by ~9.5 (log2 units) three times, "jump" by ~420 at once after the first tile,
# "falling" never.
LARGE_SCHEDULES = {
    "rising": [7.5, 7.5, 7.5, 5.0, 5.0, 5.0, 2.5, 2.5, 2.5, 0.0, 0.0, 0.0],
    "falling": [0.0, 0.0, 0.0, 2.5, 2.5, 2.5, 5.0, 5.0, 5.0, 7.5, 7.5, 7.5],
    "jump": [110.0] + [0.0] * 11,
}


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("schedule", list(LARGE_SCHEDULES))
def test_attention_moving_maximum(schedule, dtype, paged):
    """Online softmax while a row's largest score moves between key tiles by far more than
    the tile-local range: the running reference and every accumulator are rescaled (by
    factors down to 2^-420 in "jump"), or later tiles carry weights that vanish.  The keys
    that hold the weight score near zero, so bf16 operands keep their usual accuracy (a
    score's bf16 error grows with its size, about |s| 2^-9, which only the keys of
    negligible weight reach here).  Summary page, "Tree Attention" step 3: still the softmax
    over the allowed keys, which the float64 oracle computes."""
    import medusa_tree_verification_heads_amd as mdt
    bf16 = dtype == "bf16"
    H, Dh = (2, 128) if bf16 else (2, 32)
    cs = np.array(LARGE_SCHEDULES[schedule], dtype=np.float32)
    ot = otree.cartesian_tree((3, 2))
    T = ot.T
    L = np.array([700, 333], dtype=np.int32)
    B = len(L)
    note(f"attention moving maximum {schedule} {dtype} paged={paged} T={T} prefixes={L.tolist()}")
    rng = np.random.default_rng(43 + 2 * bf16 + paged + 7 * list(LARGE_SCHEDULES).index(schedule))
    m = Dh // 2 - 1   # the slowest rotary pair is (m, m + Dh/2)

    def cast(x):
        return f32_to_bf16_bits(x) if bf16 else x

    qf = rng.standard_normal((B, T, H, Dh)).astype(np.float32)
    qf[..., m], qf[..., m + Dh // 2] = 30.0, 0.0
    q = cast(qf)
    k, v = (_draw(rng, (B, T, H, Dh), 0.5, bf16) for _ in range(2))
    page = 16

    def cache_keys(shape, slot_pos):
        x = rng.standard_normal(shape).astype(np.float32) * 0.5
        x[..., m] = -cs[np.minimum(slot_pos // 64, len(cs) - 1)][..., None]
        x[..., m + Dh // 2] = 0.0
        return cast(x)

    if paged:
        npg = [-(-int(L[b]) // page) for b in range(B)]
        pool = sum(npg) + 2
        perm = rng.permutation(pool)
        pt = np.full((B, max(npg)), -1, dtype=np.int32)
        pos = np.zeros((pool, page), dtype=np.int64)   # sequence position of each pool row
        o = 0
        for b in range(B):
            pt[b, :npg[b]] = perm[o:o + npg[b]]
            for j in range(npg[b]):
                pos[perm[o + j]] = j * page + np.arange(page)
            o += npg[b]
        Kc = cache_keys((pool, page, H, Dh), pos)
        Vc = _draw(rng, (pool, page, H, Dh), 1.0, bf16)
    else:
        pt = None
        cap = int(L.max()) + 3
        Kc = cache_keys((B, cap, H, Dh), np.broadcast_to(np.arange(cap), (B, cap)))
        Vc = _draw(rng, (B, cap, H, Dh), 1.0, bf16)
    tree = mdt.Tree.cartesian((3, 2))
    cache = mdt.KVCache(_dev(Kc), _dev(Vc), None if pt is None else torch.from_numpy(pt).cuda(), page)
    out, k_rot = mdt.tree_attention(_dev(q), _dev(k), _dev(v), cache, torch.from_numpy(L).cuda(),
                                    tree.to_device("cuda"))
    torch.cuda.synchronize()
    ro, rk = ostep.tree_attention(q, k, v, Kc, Vc, L, ot, 10000.0, bf16_store=bf16, page_table=pt, page_size=page)
    go = ostep.to_f64(_host(out))
    assert np.all(np.isfinite(go))
    eo, ek = rel_err_rows(go, ro), rel_err_rows(ostep.to_f64(_host(k_rot)), rk)
    note(f"  o rel err {eo:.2e}, k_rot rel err {ek:.2e}")
    assert eo <= REL_TOL and ek <= REL_TOL
