"""Host-side tests of libmdt (CPU only): exports, tree builders, argument validation.

No kernel is launched here: every call below fails validation before any launch.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import medusa_tree_verification_heads_amd as mdt
from oracle import tree as ot
from workloads.configs import PARITY_CASES, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mdt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mdt_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "mdt_medusa_heads" in names and "mdt_kv_compact" in names
    for n in names:
        assert hasattr(mdt.lib, n), n
    assert set(names) == set(mdt.EXPORTED)


def test_abi_and_strings():
    assert mdt.lib.mdt_abi_version() == 1
    assert mdt.lib.mdt_status_string(0) == b"ok"
    assert mdt.lib.mdt_status_string(-2) == b"bad shape"


def _same_tree(lib_tree, o):
    assert lib_tree.T == o.T
    assert list(lib_tree.parent) == o.parent
    assert list(lib_tree.depth) == o.depth
    assert list(lib_tree.rank) == o.rank
    assert lib_tree.max_depth == o.max_depth
    M = ot.ancestor_mask(o)
    for i in range(o.T):
        bits = [(int(lib_tree.anc[i, j // 64]) >> (j % 64)) & 1 for j in range(o.T)]
        assert bits == [int(x) for x in M[i]]


@pytest.mark.parametrize("s", [(), (1,), (3, 2), (2, 3), (4, 2, 2), (8, 8), (1, 1, 1, 1, 1)])
def test_cartesian_matches_oracle(s):
    _same_tree(mdt.Tree.cartesian(s), ot.cartesian_tree(s))


@pytest.mark.parametrize("K,k,T", [(4, 10, 64), (5, 10, 64), (4, 10, 42), (5, 16, 256), (2, 3, 9), (3, 6, 40),
                                   (1, 32, 33), (8, 2, 200)])
def test_scored_matches_oracle(K, k, T):
    _same_tree(mdt.Tree.scored(K, k, T), ot.scored_tree_greedy(K, k, T))


def test_scored_alternative_bases_match_oracle():
    _same_tree(mdt.Tree.scored(4, 10, 64, depth_base=1), ot.scored_tree_greedy(4, 10, 64, depth_base=1))
    _same_tree(mdt.Tree.scored(4, 10, 64, rank_base=1), ot.scored_tree_greedy(4, 10, 64, rank_base=1))


def test_workload_trees_match_oracle():
    for w in list(WORKLOADS.values()) + list(PARITY_CASES.values()):
        _same_tree(mdt.Tree.for_workload(w), ot.build_tree(w))


def test_tree_builder_errors():
    h = mdt.TreeHost()
    assert mdt.lib.mdt_tree_build_scored(4, 10, 0, 0.6, 0.7, 0.8, 0, 0, ctypes.byref(h)) == -2
    assert mdt.lib.mdt_tree_build_scored(4, 10, 64, 1.5, 0.7, 0.8, 0, 0, ctypes.byref(h)) == -6
    assert mdt.lib.mdt_tree_build_scored(2, 2, 8, 0.6, 0.7, 0.8, 0, 0, ctypes.byref(h)) == -2   # only 6 candidates
    s = (ctypes.c_int * 2)(16, 16)
    assert mdt.lib.mdt_tree_build_cartesian(2, s, ctypes.byref(h)) == -2                      # 273 > 256 nodes
    assert mdt.lib.mdt_tree_build_cartesian(1, None, ctypes.byref(h)) == -1
    assert b"" != mdt.lib.mdt_last_error()


# ---------------------------------------------------------------- validation (no launch)

P = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p((1 << 20) + 2)


def _tree_desc():
    t = mdt.Tree.scored(4, 10, 64)
    d = mdt.TreeDev()
    d.T, d.max_depth, d.max_rank, d.anc_words = t.T, t.max_depth, t.max_rank, t.anc_words
    d.parent = d.depth = d.rank = d.anc = 1 << 20
    return d


def test_heads_validation():
    f = mdt.lib.mdt_medusa_heads
    def call(dt=1, B=1, d=4096, V=32000, K=4, h=P, W1=P, W2=P, Wlm=P, out=P, ws=P, nb=1 << 30):
        return f(None, dt, B, d, V, K, h, W1, W2, Wlm, out, ws, nb)
    assert call(dt=7) == -3
    assert call(d=4095) == -2
    assert call(K=0) == -2 and call(K=9) == -2
    assert call(V=0) == -2
    assert call(h=None) == -1
    assert call(W2=MIS) == -4
    assert call(ws=None) == -7
    assert call(nb=100) == -7


def test_topk_validation():
    d = _tree_desc()
    f = mdt.lib.mdt_topk_tree_expand
    def call(B=1, K=4, V=32000, k=10, tree=d, nb=1 << 30, logits=P):
        return f(None, B, K, V, k, logits, ctypes.byref(tree) if tree is not None else None, P, P, P, P, P, P, nb)
    assert call(k=0) == -2 and call(k=33) == -2
    assert call(K=3) == -5            # tree depth 4 > K
    assert call(k=8) == -5            # tree uses rank 8
    assert call(tree=None) == -1
    assert call(logits=None) == -1
    assert call(nb=4) == -7
    assert call(V=1 << 20, k=32) == -9


def test_attention_validation():
    d = _tree_desc()
    c = mdt.KVCacheDesc()
    c.layout, c.capacity, c.k, c.v = 0, 1029, 1 << 20, 1 << 20
    f = mdt.lib.mdt_tree_attention
    def call(dt=1, Dh=128, theta=10000.0, cache=c, q=P):
        return f(None, dt, 1, 32, Dh, ctypes.byref(d), q, P, P, ctypes.byref(cache), P, theta, P, P, P, 1 << 30)
    assert call(Dh=64) == -9
    assert call(dt=0, Dh=3) == -2
    assert call(theta=0.0) == -6
    assert call(q=MIS) == -4
    pc = mdt.KVCacheDesc()
    pc.layout, pc.capacity, pc.page_size, pc.max_pages, pc.num_pages = 1, 1000, 16, 64, 10
    pc.k, pc.v, pc.page_table = 1 << 20, 1 << 20, 1 << 20
    assert call(cache=pc) == -2       # capacity != max_pages * page_size
    bad = mdt.KVCacheDesc()
    bad.layout, bad.capacity, bad.k, bad.v = 5, 10, 1 << 20, 1 << 20
    assert call(cache=bad) == -6


def test_verify_accept_compact_validation():
    d = _tree_desc()
    v = mdt.lib.mdt_verify_logits
    assert v(None, 1, 1, 63, 4096, 32000, P, P, ctypes.byref(d), P, 0.0, P, P, None, P, 1 << 30) == -2   # T mismatch
    assert v(None, 1, 1, 64, 4008, 32000, P, P, ctypes.byref(d), P, 0.0, P, P, None, P, 1 << 30) == -2   # d % 32
    assert v(None, 1, 1, 64, 4096, 32000, P, P, ctypes.byref(d), P, -1.0, P, P, None, P, 1 << 30) == -6
    assert v(None, 1, 1, 64, 4096, 32000, P, P, ctypes.byref(d), P, 0.7, P, P, None, P, 16) == -7
    a = mdt.lib.mdt_accept_path
    assert a(None, 1, ctypes.byref(d), P, P, P, 3, 0.09, 0.3, 0.7, P, 5, P) == -6        # mode
    assert a(None, 1, ctypes.byref(d), P, P, P, 1, 0.0, 0.3, 0.7, P, 5, P) == -6         # eps
    assert a(None, 1, ctypes.byref(d), P, P, P, 0, 0.09, 0.3, 0.0, P, 4, P) == -2        # stride < depth+1
    k = mdt.lib.mdt_kv_compact
    c = mdt.KVCacheDesc()
    c.layout, c.capacity, c.k, c.v = 0, 1029, 1 << 20, 1 << 20
    assert k(None, 1, 1, 64, 3, 5, P, 5, P, P, P, ctypes.byref(c), P, P) == -2           # row not 16-byte multiple
    assert k(None, 2, 1, 64, 32, 128, P, 5, P, P, P, ctypes.byref(c), P, P) == -3
    ac = mdt.lib.mdt_accept_compact
    def fused(dt=1, H=32, Dh=128, mode=1, eps=0.09, stride=5, cache=c, kr=P):
        return ac(None, dt, 1, H, Dh, ctypes.byref(d), P, P, P, mode, eps, 0.3, 0.7, P, stride, P, kr, P,
                  ctypes.byref(cache), P, P)
    assert fused(mode=3) == -6 and fused(eps=0.0) == -6      # the accept_path checks
    assert fused(stride=4) == -2
    assert fused(dt=1, H=1, Dh=3) == -2                       # the kv_compact checks
    assert fused(dt=2) == -3
    assert fused(kr=None) == -1 and fused(kr=MIS) == -4
    vac = mdt.lib.mdt_verify_accept_compact
    def tail(T=64, d=4096, tau=0.7, mode=1, eps=0.09, stride=5, H=32, Dh=128, dt=1, kr=P, nb=1 << 30):
        return vac(None, dt, 1, T, d, 32000, H, Dh, P, P, ctypes.byref(d_), P, tau, mode, eps, 0.3, P, P, None, P,
                   stride, P, kr, P, ctypes.byref(c), P, P, P, nb)
    d_ = d
    assert tail(mode=3) == -6 and tail(eps=0.0) == -6 and tail(stride=4) == -2   # the accept_path checks
    assert tail(H=1, Dh=3) == -2 and tail(kr=None) == -1                          # the kv_compact checks
    assert tail(T=63) == -2 and tail(d=4008) == -2 and tail(tau=-1.0) == -6       # the verify_logits checks
    assert tail(nb=16) == -7


def test_next_state_and_rejection_validation():
    n = mdt.lib.mdt_next_state
    assert n(None, 3, 1, 64, 4096, P, P, 5, P, P) == -3          # dtype
    assert n(None, 1, 1, 64, 4093, P, P, 5, P, P) == -2          # row not a 16-byte multiple
    assert n(None, 1, 1, 64, 4096, P, P, 0, P, P) == -2          # path_stride
    assert n(None, 1, 1, 64, 4096, None, P, 5, P, P) == -1
    assert n(None, 1, 1, 64, 4096, MIS, P, 5, P, P) == -4
    nl = mdt.lib.mdt_next_logits
    Z, O = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 30)    # non-overlapping stand-ins, never dereferenced
    assert nl(None, 1, 0, 32000, 4, Z, P, 5, P, O) == -2           # T
    assert nl(None, 1, 64, 32000, 0, Z, P, 5, P, O) == -2          # K
    assert nl(None, 1, 64, 32000, 4, Z, P, 0, P, O) == -2          # path_stride
    assert nl(None, 1, 64, 32000, 4, None, P, 5, P, O) == -1
    assert nl(None, 1, 64, 32000, 4, Z, P, 5, P, ctypes.c_void_p((1 << 20) + 4096)) == -6   # overlap
    d = _tree_desc()
    r = mdt.lib.mdt_accept_rejection
    def rej(B=1, V=32000, K=4, tau=0.7, stride=5, vl=P):
        return r(None, B, V, K, ctypes.byref(d), vl, P, P, tau, P, P, P, stride, P, P)
    assert rej(tau=0.0) == -6 and rej(tau=-1.0) == -6          # temperature must be > 0
    assert rej(V=40000) == -9                                   # vocabulary beyond one workgroup's registers
    assert rej(K=3) == -5                                       # tree deeper than K
    assert rej(stride=4) == -2 and rej(stride=1100) == -2
    assert rej(vl=None) == -1


def test_layer_calls_validation():
    """Argument errors of the decoder-layer calls come back before anything is launched."""
    L = mdt.lib
    lin = lambda M=64, N=4096, K=4096, x=P, W=P, res=None, nseg=1, act=0, y=P: \
        L.mdt_linear(None, M, N, K, x, W, res, nseg, act, y)
    assert lin(K=4008) == -2                      # K not a multiple of 32
    assert lin(N=4095) == -2                      # N not a multiple of 8
    assert lin(M=0) == -2
    assert lin(act=2) == -6                       # unknown activation
    assert lin(x=None) == -1
    assert lin(W=MIS) == -4
    assert lin(act=1, N=4112) == -2               # SwiGLU needs N % 32 == 0
    assert lin(act=1, res=P) == -6                # SwiGLU takes no residual
    assert lin(nseg=3, N=4096) == -2              # segments must divide N into multiples of 8
    assert lin(nseg=2, res=P) == -6               # residual needs one segment
    sp = lambda K=4096, n=8, x=P, part=P: L.mdt_linear_split(None, 64, 4096, K, x, P, n, part)
    assert sp(n=0) == -6 and sp(n=65) == -6
    assert sp(K=64, n=3) == -6                    # more slices than 32-wide k-steps
    assert sp(K=4096, n=33) == -6                 # rounding to 32-multiples leaves 32 slices
    assert sp(part=None) == -1
    rn = L.mdt_rmsnorm
    assert rn(None, 64, 4100, P, P, 1e-6, P) == -2
    assert rn(None, 64, 4096, P, P, -1.0, P) == -6
    assert rn(None, 64, 4096, None, P, 1e-6, P) == -1
    arn = L.mdt_add_rmsnorm
    assert arn(None, 64, 4096, 0, P, P, P, 1e-6, P) == -6   # at least one slice
    assert arn(None, 64, 4096, 2, P, P, P, 1e-6, P) == -6   # slices overlapping x
    em = L.mdt_embed
    assert em(None, 64, 4096, 0, P, P, P) == -2
    assert em(None, 64, 4096, 32000, None, P, P) == -1
    assert em(None, 64, 4096, 32000, P, MIS, P) == -4


def test_compact_layers_validation():
    c = mdt.KVCacheDesc()
    c.layout, c.capacity, c.k, c.v = 0, 1029, 1 << 20, 1 << 20
    f = lambda n=2, ks=64 * 4096, vs=64 * 4096, cs=1029 * 4096: mdt.lib.mdt_kv_compact_layers(
        None, 1, n, 1, 64, 32, 128, P, 5, P, P, ks, P, vs, ctypes.byref(c), cs, P, P)
    assert f(n=0) == -2
    assert f(ks=64 * 4096 - 8) == -2              # stride smaller than one layer
    assert f(cs=1029 * 4096 - 8) == -2
    assert f(vs=-8) == -4 and f(ks=3) == -4       # negative or not a 16-byte multiple


def test_unknown_mode_strings_are_rejected():
    """A typo in the acceptance mode must not silently run typical acceptance, and the chain
    refuses rejection sampling (its sampled next token has no place in the chain)."""
    from medusa_tree_verification_heads_amd.step import DecodeLoop, VerifyStep
    w = PARITY_CASES["7b-mini"]
    for bad in ("greedly", "Typical", "rejection_sampling", ""):
        with pytest.raises(ValueError):
            VerifyStep(w, {}, mode=bad)
    with pytest.raises(ValueError):
        DecodeLoop(w, {}, [], mode="rejection")


def test_noalloc_heads_rejects_oversize():
    """The allocation-free heads call refuses activations beyond its fixed device array
    before any HIP call."""
    assert mdt.lib.mdt_medusa_heads_noalloc(None, mdt.MDT_BF16, 9, 16384, 32000, 8, 16, 16, 16, 16, 16) == -7
    assert b"exceeds the fixed scratch" in mdt.lib.mdt_last_error()
    assert mdt.lib.mdt_medusa_heads_noalloc(None, mdt.MDT_BF16, 0, 4096, 32000, 4, 16, 16, 16, 16, 16) == -2
