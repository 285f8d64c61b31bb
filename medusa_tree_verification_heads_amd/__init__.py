"""Python binding of libmdt, the MI355X (gfx950) Medusa draft-and-verify step.

Argument marshalling only: every computation runs in the HIP kernels of
``libmdt.so``.  Tensors are torch CUDA (HIP) tensors; the binding passes their
device pointers and the current torch stream to the C ABI declared in
``include/mdt.h``.  The functions carry the C names without the ``mdt_`` prefix:

    medusa_heads, topk_tree_expand, tree_attention, verify_logits,
    accept_path, kv_compact, accept_compact (the last two in one launch),
    next_state (the hidden state a following step starts from),
    accept_rejection (rejection-sampling acceptance)

plus the static tree helpers (``Tree``) and workspace queries.  Importing this
module without a built ``libmdt.so`` raises ImportError: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MDT_LIB_PATH selects another build of the library (the host-sanitizer test loads the
# host-only ASan/UBSan build this way)
LIB_PATH = os.environ.get("MDT_LIB_PATH") or os.path.join(_PKG, "libmdt.so")

MDT_F32, MDT_BF16 = 0, 1
GREEDY, TYPICAL = 0, 1
KV_CONTIG, KV_PAGED = 0, 1
MAX_NODES, MAX_HEADS, MAX_TOPK = 256, 8, 32

c_int, c_i32, c_size, c_void_p, c_float, c_double = (ctypes.c_int, ctypes.c_int32, ctypes.c_size_t,
                                                      ctypes.c_void_p, ctypes.c_float, ctypes.c_double)


class TreeHost(ctypes.Structure):
    _fields_ = [("T", c_i32), ("max_depth", c_i32), ("max_rank", c_i32), ("anc_words", c_i32),
                ("parent", ctypes.POINTER(c_i32)), ("depth", ctypes.POINTER(c_i32)),
                ("rank", ctypes.POINTER(c_i32)), ("anc", ctypes.POINTER(ctypes.c_uint64))]


class TreeDev(ctypes.Structure):
    _fields_ = [("T", c_i32), ("max_depth", c_i32), ("max_rank", c_i32), ("anc_words", c_i32),
                ("parent", c_void_p), ("depth", c_void_p), ("rank", c_void_p), ("anc", c_void_p)]


class KVCacheDesc(ctypes.Structure):
    _fields_ = [("layout", c_i32), ("capacity", c_i32), ("page_size", c_i32), ("max_pages", c_i32),
                ("num_pages", c_i32), ("reserved", c_i32), ("k", c_void_p), ("v", c_void_p),
                ("page_table", c_void_p)]


# mdt_row_stats as a numpy record (16 bytes)
ROW_STATS_DTYPE = np.dtype([("max", np.float32), ("argmax", np.int32), ("logZ", np.float32), ("entropy", np.float32)])

# (name, restype, argtypes)
_SIGS = [
    ("mdt_abi_version", c_int, []),
    ("mdt_profile_attach", c_int, [ctypes.POINTER(c_void_p), c_int]),
    ("mdt_profile_detach", c_int, []),
    ("mdt_profile_kernel", ctypes.c_char_p, [c_int]),
    ("mdt_status_string", ctypes.c_char_p, [c_int]),
    ("mdt_last_error", ctypes.c_char_p, []),
    ("mdt_tree_build_cartesian", c_int, [c_int, ctypes.POINTER(c_int), ctypes.POINTER(TreeHost)]),
    ("mdt_tree_build_scored", c_int, [c_int, c_int, c_int, c_double, c_double, c_double, c_int, c_int,
                                      ctypes.POINTER(TreeHost)]),
    ("mdt_tree_build_table", c_int, [c_int, c_int, c_int, ctypes.POINTER(c_double), ctypes.POINTER(TreeHost)]),
    ("mdt_tree_expected_length", c_int, [ctypes.POINTER(TreeHost), c_int, c_int, ctypes.POINTER(c_double),
                                         ctypes.POINTER(c_double)]),
    ("mdt_tree_free", None, [ctypes.POINTER(TreeHost)]),
    ("mdt_tree_image_bytes", c_size, [c_int]),
    ("mdt_tree_pack", c_int, [ctypes.POINTER(TreeHost), c_void_p, c_size]),
    ("mdt_tree_dev_init", c_int, [ctypes.POINTER(TreeHost), c_void_p, ctypes.POINTER(TreeDev)]),
    ("mdt_medusa_heads_workspace", c_size, [c_int, c_int, c_int]),
    ("mdt_medusa_heads", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_size]),
    ("mdt_medusa_heads_noalloc", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p]),
    ("mdt_topk_workspace", c_size, [c_int, c_int, c_int, c_int]),
    ("mdt_topk_tree_expand", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, ctypes.POINTER(TreeDev),
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size]),
    ("mdt_tree_attention_workspace", c_size, [c_int, c_int, c_int, c_int, c_int, c_int]),
    ("mdt_tree_attention", c_int, [c_void_p, c_int, c_int, c_int, c_int, ctypes.POINTER(TreeDev), c_void_p,
                                   c_void_p, c_void_p, ctypes.POINTER(KVCacheDesc), c_void_p, c_float, c_void_p,
                                   c_void_p, c_void_p, c_size]),
    ("mdt_verify_logits_workspace", c_size, [c_int, c_int, c_int, c_int, c_int]),
    ("mdt_verify_logits", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                  ctypes.POINTER(TreeDev), c_void_p, c_float, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_size]),
    ("mdt_accept_path", c_int, [c_void_p, c_int, ctypes.POINTER(TreeDev), c_void_p, c_void_p, c_void_p, c_int,
                                c_float, c_float, c_float, c_void_p, c_int, c_void_p]),
    ("mdt_kv_compact", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p,
                               c_void_p, ctypes.POINTER(KVCacheDesc), c_void_p, c_void_p]),
    ("mdt_accept_compact", c_int, [c_void_p, c_int, c_int, c_int, c_int, ctypes.POINTER(TreeDev), c_void_p, c_void_p,
                                   c_void_p, c_int, c_float, c_float, c_float, c_void_p, c_int, c_void_p, c_void_p,
                                   c_void_p, ctypes.POINTER(KVCacheDesc), c_void_p, c_void_p]),
    ("mdt_verify_accept_compact", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p,
                                          c_void_p, ctypes.POINTER(TreeDev), c_void_p, c_float, c_int, c_float,
                                          c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p,
                                          c_void_p, ctypes.POINTER(KVCacheDesc), c_void_p, c_void_p, c_void_p,
                                          c_size]),
    ("mdt_next_state", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p,
                               c_void_p]),
    ("mdt_next_logits", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p,
                                c_void_p]),
    ("mdt_accept_rejection", c_int, [c_void_p, c_int, c_int, c_int, ctypes.POINTER(TreeDev), c_void_p, c_void_p,
                                     c_void_p, c_float, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p]),
    ("mdt_kv_compact_layers", c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_int, c_void_p,
                                      c_void_p, ctypes.c_longlong, c_void_p, ctypes.c_longlong,
                                      ctypes.POINTER(KVCacheDesc), ctypes.c_longlong, c_void_p, c_void_p]),
    ("mdt_embed", c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    ("mdt_rmsnorm", c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_float, c_void_p]),
    ("mdt_add_rmsnorm", c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_float, c_void_p]),
    ("mdt_linear", c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p]),
    ("mdt_linear_split", c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p]),
]

EXPORTED = [name for name, _, _ in _SIGS]


def _mapped_hip_runtimes():
    libs = set()
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1] if line.strip() else ""
            if "libamdhip64" in path:
                libs.add(os.path.realpath(path))
    return libs


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m medusa_tree_verification_heads_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in _SIGS:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    rts = _mapped_hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"libmdt and torch bind different HIP runtimes: {sorted(rts)}")
    return lib


lib = _load()


class MdtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.mdt_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.mdt_status_string(status).decode()} ({status}): {msg}")


def _check(st: int, where: str):
    if st != 0:
        raise MdtError(st, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MDT_BF16
    if t.dtype == torch.float32:
        return MDT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace buffer (zero-filled so that its contents are deterministic)."""
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def _ws(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    t = new_workspace(nbytes, device)
    return t, t.numel()


# ---------------------------------------------------------------------------
# static tree
# ---------------------------------------------------------------------------

class Tree:
    """A static candidate tree built by libmdt (host), with its packed image."""

    def __init__(self, host: TreeHost):
        self._host = host
        T = host.T
        self.T = T
        self.max_depth = host.max_depth
        self.max_rank = host.max_rank
        self.anc_words = host.anc_words
        self.parent = np.ctypeslib.as_array(host.parent, shape=(T,)).copy()
        self.depth = np.ctypeslib.as_array(host.depth, shape=(T,)).copy()
        self.rank = np.ctypeslib.as_array(host.rank, shape=(T,)).copy()
        self.anc = np.ctypeslib.as_array(host.anc, shape=(T * host.anc_words,)).copy().reshape(T, host.anc_words)
        n = lib.mdt_tree_image_bytes(T)
        self.image = np.zeros(n, dtype=np.uint8)
        _check(lib.mdt_tree_pack(ctypes.byref(host), self.image.ctypes.data_as(c_void_p), n), "tree_pack")

    def __del__(self):
        try:
            lib.mdt_tree_free(ctypes.byref(self._host))
        except Exception:
            pass

    @classmethod
    def cartesian(cls, s: Sequence[int]) -> "Tree":
        h = TreeHost()
        arr = (c_int * max(1, len(s)))(*s)
        _check(lib.mdt_tree_build_cartesian(len(s), arr, ctypes.byref(h)), "tree_build_cartesian")
        return cls(h)

    @classmethod
    def scored(cls, K: int, k_cfg: int, T: int, a0=0.6, rho=0.7, gamma=0.8, rank_base=0, depth_base=0) -> "Tree":
        h = TreeHost()
        _check(lib.mdt_tree_build_scored(K, k_cfg, T, a0, rho, gamma, rank_base, depth_base, ctypes.byref(h)),
               "tree_build_scored")
        return cls(h)

    @classmethod
    def from_table(cls, acc, T: int) -> "Tree":
        """Sparse tree of T nodes from an accuracy table acc [K][k] (rank-r accuracy of head j+1)."""
        a = np.ascontiguousarray(acc, dtype=np.float64)
        K, k = a.shape
        h = TreeHost()
        _check(lib.mdt_tree_build_table(K, k, T, a.ctypes.data_as(ctypes.POINTER(c_double)), ctypes.byref(h)),
               "tree_build_table")
        return cls(h)

    def expected_length(self, acc) -> float:
        """E[L] of this tree under an accuracy table acc [K][k]."""
        a = np.ascontiguousarray(acc, dtype=np.float64)
        out = c_double()
        _check(lib.mdt_tree_expected_length(ctypes.byref(self._host), a.shape[0], a.shape[1],
                                            a.ctypes.data_as(ctypes.POINTER(c_double)), ctypes.byref(out)),
               "tree_expected_length")
        return out.value

    @classmethod
    def for_workload(cls, w) -> "Tree":
        if w.tree_kind == "cartesian":
            return cls.cartesian(w.tree_s)
        return cls.scored(w.K, w.k_cfg, w.T, w.a0, w.rho, w.gamma)

    def to_device(self, device="cuda") -> "DeviceTree":
        return DeviceTree(self, device)


class DeviceTree:
    """Device copy of a tree's packed image and the mdt_tree_dev describing it."""

    def __init__(self, tree: Tree, device):
        self.tree = tree
        self.image = torch.from_numpy(tree.image).to(device)
        self.desc = TreeDev()
        _check(lib.mdt_tree_dev_init(ctypes.byref(tree._host), c_void_p(self.image.data_ptr()),
                                     ctypes.byref(self.desc)), "tree_dev_init")

    @property
    def T(self):
        return self.tree.T


class KVCache:
    """Caller-owned prefix cache: contiguous [B][capacity][H][Dh] or paged pool + page table."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, page_table: Optional[torch.Tensor] = None,
                 page_size: int = 16):
        self.k, self.v, self.page_table = k, v, page_table
        d = KVCacheDesc()
        if page_table is None:
            d.layout = KV_CONTIG
            d.capacity = k.shape[1]
        else:
            d.layout = KV_PAGED
            d.page_size = page_size
            d.max_pages = page_table.shape[1]
            d.num_pages = k.shape[0]
            d.capacity = d.max_pages * page_size
            d.page_table = page_table.data_ptr()
        d.k = k.data_ptr()
        d.v = v.data_ptr()
        self.desc = d


# ---------------------------------------------------------------------------
# the six calls
# ---------------------------------------------------------------------------

def medusa_heads_workspace(B, d, K) -> int:
    return lib.mdt_medusa_heads_workspace(B, d, K)


def medusa_heads(h, W1, W2, Wlm, logits=None, ws=None, stream=None):
    """logits[b][0] = Wlm h_b; logits[b][k] = W2_k (SiLU(W1_k h_b) + h_b).  Wlm None:
    slot 0 is left as it is."""
    B, d = h.shape
    K, V = W1.shape[0], W2.shape[1]
    if logits is None:
        logits = torch.empty((B, K + 1, V), dtype=torch.float32, device=h.device)
    ws, nb = _ws(medusa_heads_workspace(B, d, K), h.device, ws)
    _check(lib.mdt_medusa_heads(_stream(stream), _dtype_code(h), B, d, V, K, _ptr(h), _ptr(W1), _ptr(W2), _ptr(Wlm),
                                _ptr(logits), _ptr(ws), nb), "medusa_heads")
    return logits


HEADS_NOALLOC_MAX_BYTES = 4 << 20


def medusa_heads_noalloc(h, W1, W2, Wlm, logits, stream=None):
    """medusa_heads with the activations in the library's fixed device array (no workspace,
    nothing allocated; ``logits`` must be given).  Calls overlapping on one GPU race."""
    B, d = h.shape
    K, V = W1.shape[0], W2.shape[1]
    _check(lib.mdt_medusa_heads_noalloc(_stream(stream), _dtype_code(h), B, d, V, K, _ptr(h), _ptr(W1), _ptr(W2),
                                        _ptr(Wlm), _ptr(logits)), "medusa_heads_noalloc")
    return logits


def topk_workspace(B, K, V, k_cfg) -> int:
    return lib.mdt_topk_workspace(B, K, V, k_cfg)


def topk_tree_expand(logits, k_cfg: int, tree: DeviceTree, prefix_len, topk_idx=None, topk_val=None,
                     tree_tokens=None, pos_ids=None, ws=None, stream=None):
    B, K1, V = logits.shape
    dev = logits.device
    T = tree.T
    topk_idx = torch.empty((B, K1, k_cfg), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_val = torch.empty((B, K1, k_cfg), dtype=torch.float32, device=dev) if topk_val is None else topk_val
    tree_tokens = torch.empty((B, T), dtype=torch.int32, device=dev) if tree_tokens is None else tree_tokens
    pos_ids = torch.empty((B, T), dtype=torch.int32, device=dev) if pos_ids is None else pos_ids
    ws, nb = _ws(topk_workspace(B, K1 - 1, V, k_cfg), dev, ws)
    _check(lib.mdt_topk_tree_expand(_stream(stream), B, K1 - 1, V, k_cfg, _ptr(logits), ctypes.byref(tree.desc),
                                    _ptr(prefix_len), _ptr(topk_idx), _ptr(topk_val), _ptr(tree_tokens),
                                    _ptr(pos_ids), _ptr(ws), nb), "topk_tree_expand")
    return topk_idx, topk_val, tree_tokens, pos_ids


def tree_attention_workspace(dtype_code, B, T, H, Dh, capacity) -> int:
    return lib.mdt_tree_attention_workspace(dtype_code, B, T, H, Dh, capacity)


def tree_attention(q, k, v, cache: KVCache, prefix_len, tree: DeviceTree, rope_theta=10000.0, out=None, k_rot=None,
                   ws=None, stream=None):
    B, T, H, Dh = q.shape
    out = torch.empty_like(q) if out is None else out
    k_rot = torch.empty_like(k) if k_rot is None else k_rot
    dt = _dtype_code(q)
    ws, nb = _ws(tree_attention_workspace(dt, B, T, H, Dh, cache.desc.capacity), q.device, ws)
    _check(lib.mdt_tree_attention(_stream(stream), dt, B, H, Dh, ctypes.byref(tree.desc), _ptr(q), _ptr(k), _ptr(v),
                                  ctypes.byref(cache.desc), _ptr(prefix_len), float(rope_theta), _ptr(out),
                                  _ptr(k_rot), _ptr(ws), nb), "tree_attention")
    return out, k_rot


def verify_logits_workspace(dtype_code, B, T, d, V) -> int:
    return lib.mdt_verify_logits_workspace(dtype_code, B, T, d, V)


def verify_logits(x, Wlm, tree: DeviceTree, tree_tokens, temperature: float, stats=None, edge=None,
                  want_logits=False, logits=None, ws=None, stream=None):
    """x [B*T][d]; returns (stats as int32 [B*T][4] view, edge [B][T], logits or None)."""
    M, d = x.shape
    V = Wlm.shape[0]
    T = tree.T
    B = M // T
    dev = x.device
    stats = torch.empty((M, 4), dtype=torch.int32, device=dev) if stats is None else stats
    edge = torch.empty((B, T), dtype=torch.float32, device=dev) if edge is None else edge
    if want_logits and logits is None:
        logits = torch.empty((M, V), dtype=torch.float32, device=dev)
    dt = _dtype_code(x)
    ws, nb = _ws(verify_logits_workspace(dt, B, T, d, V), dev, ws)
    _check(lib.mdt_verify_logits(_stream(stream), dt, B, T, d, V, _ptr(x), _ptr(Wlm), ctypes.byref(tree.desc),
                                 _ptr(tree_tokens), float(temperature), _ptr(stats), _ptr(edge), _ptr(logits),
                                 _ptr(ws), nb), "verify_logits")
    return stats, edge, logits


class KernelTimer:
    """Start/stop timing events around every kernel the library launches (on its stream).

    with KernelTimer(n_launches) as kt:  ... library calls ...
    then kt.durations_ms() -> list of (kernel name, ms between the kernel's start and end).
    """

    def __init__(self, capacity: int):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * capacity)]
        for e in self.events:      # materialise the underlying HIP events
            e.record()
        torch.cuda.synchronize()
        self._arr = (c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
        self.count = 0
        self.names = []

    def __enter__(self):
        _check(lib.mdt_profile_attach(self._arr, len(self.events)), "profile_attach")
        return self

    def __exit__(self, *exc):
        self.count = lib.mdt_profile_detach()
        n = min(self.count, len(self.events) // 2)
        self.names = [lib.mdt_profile_kernel(i).decode() for i in range(n)]
        return False

    def durations_ms(self):
        torch.cuda.synchronize()
        return [(name, self.events[2 * i].elapsed_time(self.events[2 * i + 1])) for i, name in enumerate(self.names)]


def stats_to_numpy(stats: torch.Tensor) -> np.ndarray:
    """Device mdt_row_stats buffer -> numpy record array (max, argmax, logZ, entropy)."""
    return stats.cpu().numpy().view(ROW_STATS_DTYPE).reshape(-1)


def accept_path(stats, edge, tree_tokens, tree: DeviceTree, mode: int, eps=0.09, delta=0.3, temperature=0.0,
                path=None, n_acc=None, path_stride=None, stream=None):
    B, T = tree_tokens.shape
    dev = tree_tokens.device
    path_stride = tree.tree.max_depth + 1 if path_stride is None else path_stride
    path = torch.empty((B, path_stride), dtype=torch.int32, device=dev) if path is None else path
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev) if n_acc is None else n_acc
    _check(lib.mdt_accept_path(_stream(stream), B, ctypes.byref(tree.desc), _ptr(stats), _ptr(edge),
                               _ptr(tree_tokens), int(mode), float(eps), float(delta), float(temperature),
                               _ptr(path), path_stride, _ptr(n_acc)), "accept_path")
    return path, n_acc


def kv_compact(path, n_acc, k_rot, v, cache: KVCache, prefix_len, new_prefix_len=None, stream=None):
    B, T, H, Dh = k_rot.shape
    new_prefix_len = torch.empty_like(prefix_len) if new_prefix_len is None else new_prefix_len
    _check(lib.mdt_kv_compact(_stream(stream), _dtype_code(k_rot), B, T, H, Dh, _ptr(path), path.shape[1],
                              _ptr(n_acc), _ptr(k_rot), _ptr(v), ctypes.byref(cache.desc), _ptr(prefix_len),
                              _ptr(new_prefix_len)), "kv_compact")
    return new_prefix_len


def accept_rejection(vlogits, head_logits, tree_tokens, tree: DeviceTree, temperature, u_accept, u_resample,
                     path=None, n_acc=None, next_token=None, path_stride=None, stream=None):
    """Rejection-sampling acceptance; returns (path, n_acc, next_token)."""
    B, K1, V = head_logits.shape
    ps = path_stride or tree.tree.max_depth + 1
    dev = head_logits.device
    path = torch.empty((B, ps), dtype=torch.int32, device=dev) if path is None else path
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev) if n_acc is None else n_acc
    next_token = torch.empty((B,), dtype=torch.int32, device=dev) if next_token is None else next_token
    _check(lib.mdt_accept_rejection(_stream(stream), B, V, K1 - 1, ctypes.byref(tree.desc), _ptr(vlogits),
                                    _ptr(head_logits), _ptr(tree_tokens), float(temperature), _ptr(u_accept),
                                    _ptr(u_resample), _ptr(path), path.shape[1], _ptr(n_acc), _ptr(next_token)),
           "accept_rejection")
    return path, n_acc, next_token


def next_state(x, path, n_acc, out=None, stream=None):
    """Row of x [B][T][d] at each sequence's deepest accepted node -> [B][d]."""
    B, T, d = x.shape
    out = torch.empty((B, d), dtype=x.dtype, device=x.device) if out is None else out
    _check(lib.mdt_next_state(_stream(stream), _dtype_code(x), B, T, d, _ptr(x), _ptr(path), path.shape[1],
                              _ptr(n_acc), _ptr(out)), "next_state")
    return out


def next_logits(vlogits, path, n_acc, head_logits, stream=None):
    """head_logits[b][0] = the verifier row (vlogits [B*T][V] or [B][T][V]) of sequence
    b's deepest accepted node; returns head_logits."""
    B, K1, V = head_logits.shape
    T = vlogits.numel() // (B * V)
    _check(lib.mdt_next_logits(_stream(stream), B, T, V, K1 - 1, _ptr(vlogits), _ptr(path), path.shape[1],
                               _ptr(n_acc), _ptr(head_logits)), "next_logits")
    return head_logits


def accept_compact(stats, edge, tree_tokens, tree: DeviceTree, mode: int, eps, delta, temperature, k_rot, v,
                   cache: KVCache, prefix_len, path=None, n_acc=None, new_prefix_len=None, path_stride=None,
                   stream=None):
    """accept_path then kv_compact in one launch; returns (path, n_acc, new_prefix_len)."""
    B, T, H, Dh = k_rot.shape
    dev = k_rot.device
    path_stride = tree.tree.max_depth + 1 if path_stride is None else path_stride
    path = torch.empty((B, path_stride), dtype=torch.int32, device=dev) if path is None else path
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev) if n_acc is None else n_acc
    new_prefix_len = torch.empty_like(prefix_len) if new_prefix_len is None else new_prefix_len
    _check(lib.mdt_accept_compact(_stream(stream), _dtype_code(k_rot), B, H, Dh, ctypes.byref(tree.desc), _ptr(stats),
                                  _ptr(edge), _ptr(tree_tokens), int(mode), float(eps), float(delta),
                                  float(temperature), _ptr(path), path_stride, _ptr(n_acc), _ptr(k_rot), _ptr(v),
                                  ctypes.byref(cache.desc), _ptr(prefix_len), _ptr(new_prefix_len)),
           "accept_compact")
    return path, n_acc, new_prefix_len


def verify_accept_compact(x, Wlm, tree: DeviceTree, tree_tokens, temperature: float, mode: int, eps, delta, k_rot,
                          v, cache: KVCache, prefix_len, stats=None, edge=None, logits=None, want_logits=False,
                          path=None, n_acc=None, new_prefix_len=None, path_stride=None, ws=None, stream=None):
    """verify_logits, accept_path and kv_compact in two launches; returns
    (stats, edge, logits or None, path, n_acc, new_prefix_len)."""
    M, d = x.shape
    V = Wlm.shape[0]
    B, T = tree_tokens.shape
    _, _, H, Dh = k_rot.shape
    dev = x.device
    stats = torch.empty((M, 4), dtype=torch.int32, device=dev) if stats is None else stats
    edge = torch.empty((B, T), dtype=torch.float32, device=dev) if edge is None else edge
    if want_logits and logits is None:
        logits = torch.empty((M, V), dtype=torch.float32, device=dev)
    path_stride = tree.tree.max_depth + 1 if path_stride is None else path_stride
    path = torch.empty((B, path_stride), dtype=torch.int32, device=dev) if path is None else path
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev) if n_acc is None else n_acc
    new_prefix_len = torch.empty_like(prefix_len) if new_prefix_len is None else new_prefix_len
    dt = _dtype_code(x)
    ws, nb = _ws(verify_logits_workspace(dt, B, T, d, V), dev, ws)
    _check(lib.mdt_verify_accept_compact(_stream(stream), dt, B, T, d, V, H, Dh, _ptr(x), _ptr(Wlm),
                                         ctypes.byref(tree.desc), _ptr(tree_tokens), float(temperature), int(mode),
                                         float(eps), float(delta), _ptr(stats), _ptr(edge),
                                         _ptr(logits) if want_logits else None, _ptr(path), path_stride, _ptr(n_acc),
                                         _ptr(k_rot), _ptr(v), ctypes.byref(cache.desc), _ptr(prefix_len),
                                         _ptr(new_prefix_len), _ptr(ws), nb), "verify_accept_compact")
    return stats, edge, logits if want_logits else None, path, n_acc, new_prefix_len


def kv_compact_layers(path, n_acc, k_rot, v, cache: KVCache, prefix_len, cache_layer_stride: int,
                      new_prefix_len=None, stream=None):
    """kv_compact for every layer at once: k_rot and v are [n_layers][B][T][H][Dh] views (any
    layer stride), ``cache`` describes layer 0 and layer l's rows sit cache_layer_stride
    elements further on."""
    n_layers, B, T, H, Dh = k_rot.shape
    for t in (k_rot, v):
        assert t.shape == k_rot.shape and t[0].is_contiguous(), "each layer must be a contiguous [B][T][H][Dh]"
    new_prefix_len = torch.empty_like(prefix_len) if new_prefix_len is None else new_prefix_len
    _check(lib.mdt_kv_compact_layers(_stream(stream), _dtype_code(k_rot), n_layers, B, T, H, Dh, _ptr(path),
                                     path.shape[1], _ptr(n_acc), _ptr(k_rot), k_rot.stride(0), _ptr(v), v.stride(0),
                                     ctypes.byref(cache.desc), int(cache_layer_stride), _ptr(prefix_len),
                                     _ptr(new_prefix_len)), "kv_compact_layers")
    return new_prefix_len


# ---------------------------------------------------------------------------
# decoder-layer pieces of the full verify forward (bf16)
# ---------------------------------------------------------------------------

ACT_NONE, ACT_SWIGLU = 0, 1


def _bf16_2d(t, name):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous 2-d bfloat16 tensor")


def embed(tokens, E, out=None, stream=None):
    """Rows E[tokens] -> [M][d] (a token outside the vocabulary gives a zero row)."""
    _bf16_2d(E, "E")
    M = tokens.numel()
    V, d = E.shape
    out = torch.empty((M, d), dtype=E.dtype, device=E.device) if out is None else out
    _check(lib.mdt_embed(_stream(stream), M, d, V, _ptr(tokens), _ptr(E), _ptr(out)), "embed")
    return out


def rmsnorm(x, g, eps: float, out=None, stream=None):
    """bf16(x / sqrt(mean(x^2) + eps) * g) row by row."""
    _bf16_2d(x, "x")
    M, d = x.shape
    out = torch.empty_like(x) if out is None else out
    _check(lib.mdt_rmsnorm(_stream(stream), M, d, _ptr(x), _ptr(g), float(eps), _ptr(out)), "rmsnorm")
    return out


def add_rmsnorm(part, x, g, eps: float, out=None, stream=None):
    """x += part[0] + ... + part[n-1] (fp32 sum, one bf16 rounding), in place; returns
    rmsnorm(x) * g (bf16).  part: fp32 [n][M][d]."""
    _bf16_2d(x, "x")
    M, d = x.shape
    n = part.shape[0]
    assert part.dtype == torch.float32 and part.shape == (n, M, d) and part.is_contiguous()
    out = torch.empty_like(x) if out is None else out
    _check(lib.mdt_add_rmsnorm(_stream(stream), M, d, n, _ptr(part), _ptr(x), _ptr(g), float(eps), _ptr(out)),
           "add_rmsnorm")
    return out


def linear(x, W, residual=None, nseg=1, act=ACT_NONE, out=None, stream=None):
    """x [M][K] times W [N][K] transposed (bf16 in and out, fp32 accumulation).

    act=ACT_NONE: (+ residual [M][N]) -> [M][N], or [nseg][M][N/nseg] column segments.
    act=ACT_SWIGLU: W holds gate/up rows interleaved by 16 (see interleave_gate_up) -> [M][N/2].
    """
    _bf16_2d(x, "x")
    _bf16_2d(W, "W")
    M, K = x.shape
    N = W.shape[0]
    if act == ACT_SWIGLU:
        shape = (M, N // 2)
    else:
        shape = (M, N) if nseg == 1 else (nseg, M, N // nseg)
    out = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    _check(lib.mdt_linear(_stream(stream), M, N, K, _ptr(x), _ptr(W), _ptr(residual), nseg, act, _ptr(out)),
           "linear")
    return out


def linear_split(x, W, nsplit: int, out=None, stream=None):
    """fp32 products of nsplit slices of the inner dimension -> [nsplit][M][N]."""
    _bf16_2d(x, "x")
    _bf16_2d(W, "W")
    M, K = x.shape
    N = W.shape[0]
    out = torch.empty((nsplit, M, N), dtype=torch.float32, device=x.device) if out is None else out
    _check(lib.mdt_linear_split(_stream(stream), M, N, K, _ptr(x), _ptr(W), int(nsplit), _ptr(out)), "linear_split")
    return out


def auto_split(M: int, N: int, K: int, device=None) -> int:
    """Slices for a product whose 64 x 64 output tiles are too few to fill the GPU: grow
    while the workgroups stay within one per compute unit (where the library runs the
    tile on twice as many waves, splitting each chunk's k-steps) and slices stay >= 512
    long."""
    cus = torch.cuda.get_device_properties(device or torch.cuda.current_device()).multi_processor_count
    tiles = -(-N // 64) * -(-M // 64)
    s = 1
    while tiles * (s + 1) <= cus and K // (s + 1) >= 512:
        s += 1

    def slices(n):  # slices left after rounding each to a multiple of 32
        ks = -(-(-(-K // n)) // 32) * 32
        return -(-K // ks)

    while s > 1 and slices(s) != s:
        s -= 1
    return s


def interleave_gate_up(Wg: torch.Tensor, Wu: torch.Tensor) -> torch.Tensor:
    """The [2F][K] weight layout of ACT_SWIGLU: rows 32i..32i+15 = Wg[16i..16i+15],
    rows 32i+16..32i+31 = Wu[16i..16i+15] (a row permutation of the stacked pair)."""
    F, K = Wg.shape
    assert Wu.shape == (F, K) and F % 16 == 0
    return torch.stack((Wg.reshape(F // 16, 16, K), Wu.reshape(F // 16, 16, K)), dim=1).reshape(2 * F, K).contiguous()

