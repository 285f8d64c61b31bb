"""GPU parity of acceptance and compaction on planted pass/fail patterns.

The planted cases (``tests/planted.py``, coverage pinned on the CPU in
``test_accept_planted.py``) make every accepted length from 1 to max_depth + 1
appear, put passing edges under failing ancestors and several accepted nodes at
the deepest accepted depth, on trees of one to four 64-bit mask words.
``mdt_accept_path`` and ``mdt_accept_compact`` (contiguous and paged caches) must
return the oracle's paths, lengths and cache rows bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import step as ostep
from tests.parity_util import note
from tests.test_accept_planted import MODES, TREES, oracle_tree, planted
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

H, DH, PAGE = 2, 64, 16


def _device_tree(name):
    import medusa_tree_verification_heads_amd as mdt
    t = oracle_tree(name)
    spec = TREES[name]
    g = mdt.Tree.cartesian(spec[1]) if spec[0] == "cartesian" else mdt.Tree.scored(*spec[1:])
    assert g.parent.tolist() == list(t.parent) and g.depth.tolist() == list(t.depth), name
    return g.to_device("cuda")


def _bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _dev_bf16(a):
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def _codes(mode):
    import medusa_tree_verification_heads_amd as mdt
    return mdt.GREEDY if mode == "greedy" else mdt.TYPICAL


def _inputs(tree_name, mode_name):
    case, paths, n_acc = planted(tree_name, mode_name)
    stats = torch.from_numpy(case["stats"].view(np.int32).copy()).cuda()
    edge = torch.from_numpy(case["edge"]).cuda()
    toks = torch.from_numpy(case["tokens"]).cuda()
    return case, paths, n_acc, stats, edge, toks


@pytest.mark.parametrize("mode_name", list(MODES))
@pytest.mark.parametrize("tree_name", list(TREES))
def test_accept_path_planted(tree_name, mode_name):
    import medusa_tree_verification_heads_amd as mdt
    mode, tau, eps, delta = MODES[mode_name]
    case, paths, n_acc, stats, edge, toks = _inputs(tree_name, mode_name)
    note(f"planted accept {tree_name} {mode_name} B={len(n_acc)}")
    dt = _device_tree(tree_name)
    path, n = mdt.accept_path(stats, edge, toks, dt, _codes(mode), eps, delta, tau)
    torch.cuda.synchronize()
    path, n = path.cpu().numpy(), n.cpu().numpy()
    assert n.tolist() == n_acc
    for b, p in enumerate(paths):
        assert path[b, :len(p)].tolist() == p, b
        assert np.all(path[b, len(p):] == -1), b


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("mode_name", ["greedy", "typical-t0.7"])
@pytest.mark.parametrize("tree_name", list(TREES))
def test_accept_compact_planted(tree_name, mode_name, paged):
    """The fused call: oracle path and lengths, and the oracle's compacted cache bit for bit
    (every other cache row untouched)."""
    import medusa_tree_verification_heads_amd as mdt
    mode, tau, eps, delta = MODES[mode_name]
    case, paths, n_acc, stats, edge, toks = _inputs(tree_name, mode_name)
    t = oracle_tree(tree_name)
    B, T = case["tokens"].shape
    note(f"planted accept_compact {tree_name} {mode_name} paged={paged} B={B}")
    rng = np.random.default_rng(B * T + paged)
    k_rot, v = _bf16(rng, (B, T, H, DH)), _bf16(rng, (B, T, H, DH))
    L = rng.integers(0, 40, B).astype(np.int32)
    L[0] = 0   # an empty prefix: the path starts at slot 0
    room = t.max_depth + 1
    if paged:
        npg = [-(-(int(L[b]) + room) // PAGE) for b in range(B)]
        pool = sum(npg) + 3
        perm = rng.permutation(pool)
        pt = np.full((B, max(npg)), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            pt[b, :npg[b]] = perm[o:o + npg[b]]
            o += npg[b]
        Kc, Vc = _bf16(rng, (pool, PAGE, H, DH)), _bf16(rng, (pool, PAGE, H, DH))
    else:
        pt = None
        cap = int(L.max()) + room + 5
        Kc, Vc = _bf16(rng, (B, cap, H, DH)), _bf16(rng, (B, cap, H, DH))
    Kd, Vd = _dev_bf16(Kc.copy()), _dev_bf16(Vc.copy())
    cache = mdt.KVCache(Kd, Vd, None if pt is None else torch.from_numpy(pt).cuda(), PAGE)
    dt = _device_tree(tree_name)
    path, n, new_len = mdt.accept_compact(stats, edge, toks, dt, _codes(mode), eps, delta, tau, _dev_bf16(k_rot),
                                          _dev_bf16(v), cache, torch.from_numpy(L).cuda())
    torch.cuda.synchronize()
    assert n.cpu().numpy().tolist() == n_acc
    pg = path.cpu().numpy()
    for b, p in enumerate(paths):
        assert pg[b, :len(p)].tolist() == p, b
    Kn, Vn, nl = ostep.kv_compact(Kc, Vc, k_rot, v, paths, L, pt, PAGE)
    assert new_len.cpu().numpy().tolist() == nl
    assert np.array_equal(Kd.view(torch.int16).cpu().numpy().view(np.uint16), Kn)
    assert np.array_equal(Vd.view(torch.int16).cpu().numpy().view(np.uint16), Vn)


@pytest.mark.parametrize("tree_name", ["7b-T64", "33b-T256"])
def test_separate_compact_planted(tree_name):
    """mdt_accept_path then mdt_kv_compact on the planted typical case: the oracle's cache."""
    import medusa_tree_verification_heads_amd as mdt
    mode, tau, eps, delta = MODES["typical-t0.7"]
    case, paths, n_acc, stats, edge, toks = _inputs(tree_name, "typical-t0.7")
    B, T = case["tokens"].shape
    rng = np.random.default_rng(T)
    k_rot, v = _bf16(rng, (B, T, H, DH)), _bf16(rng, (B, T, H, DH))
    L = rng.integers(1, 300, B).astype(np.int32)
    cap = int(L.max()) + oracle_tree(tree_name).max_depth + 1
    Kc, Vc = _bf16(rng, (B, cap, H, DH)), _bf16(rng, (B, cap, H, DH))
    Kd, Vd = _dev_bf16(Kc.copy()), _dev_bf16(Vc.copy())
    dt = _device_tree(tree_name)
    path, n = mdt.accept_path(stats, edge, toks, dt, _codes(mode), eps, delta, tau)
    new_len = mdt.kv_compact(path, n, _dev_bf16(k_rot), _dev_bf16(v), mdt.KVCache(Kd, Vd), torch.from_numpy(L).cuda())
    torch.cuda.synchronize()
    Kn, Vn, nl = ostep.kv_compact(Kc, Vc, k_rot, v, paths, L)
    assert n.cpu().numpy().tolist() == n_acc and new_len.cpu().numpy().tolist() == nl
    assert np.array_equal(Kd.view(torch.int16).cpu().numpy().view(np.uint16), Kn)
    assert np.array_equal(Vd.view(torch.int16).cpu().numpy().view(np.uint16), Vn)
