"""Seeded synthetic inputs for the draft-and-verify step.

Recipe (the same for every consumer):

* Every tensor has its own stream: values are drawn in fixed blocks of
  ``BLOCK`` elements, block ``j`` of tensor ``tid`` from
  ``numpy.random.Generator(PCG64(SeedSequence([seed, tid, j])))``, so the bytes
  do not depend on how many threads draw them.
* Values are N(0, s^2) with s^2 = 1/sqrt(d) (d = hidden size): standard normals
  are drawn in float32 and multiplied by s = d**-0.25 in float32.  For bf16
  workloads the float32 value is then rounded to bf16 (round to nearest, ties to
  even) and stored as its 16-bit pattern (``numpy.uint16``); fp32 workloads keep
  the float32 values.
* The prefix KV cache holds drawn values in the slots below each sequence's
  prefix length and zeros elsewhere (room for the accepted path).  Prefix keys
  stand for keys that were rotated when they were written.
* Paged caches (16-token pages): prefix lengths are uniform integers in the
  workload's inclusive range; each sequence owns ceil((L_b + K + 1)/page) pages,
  taken in order from a seeded random permutation of the physical pages; unused
  page-table entries are -1.

Nothing in this module computes any part of the step.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

BLOCK = 1 << 22

TID_H, TID_W1, TID_W2, TID_WLM, TID_KC, TID_VC, TID_Q, TID_K, TID_V, TID_LEN, TID_PAGES = range(11)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


bf16_round_bits = f32_to_bf16_bits


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _block(seed: int, tid: int, j: int, n: int, std: np.float32, bf16: bool) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, j])))
    x = rng.standard_normal(n, dtype=np.float32)
    x *= std
    return f32_to_bf16_bits(x) if bf16 else x


def normal_stream(seed: int, tid: int, count: int, std: float, bf16: bool) -> np.ndarray:
    """``count`` values of tensor ``tid`` (bf16 bit patterns or float32), in block order."""
    out = np.empty(count, dtype=np.uint16 if bf16 else np.float32)
    if count == 0:
        return out
    nblk = (count + BLOCK - 1) // BLOCK
    s = np.float32(std)

    def fill(j):
        lo = j * BLOCK
        n = min(BLOCK, count - lo)
        out[lo:lo + n] = _block(seed, tid, j, n, s, bf16)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def prefix_lengths(w: Workload, seed: int) -> np.ndarray:
    if w.L_range is None:
        return np.full(w.B, w.L, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TID_LEN])))
    lo, hi = w.L_range
    return rng.integers(lo, hi + 1, size=w.B, dtype=np.int64).astype(np.int32)


def page_layout(w: Workload, seed: int, lens: np.ndarray, steps: int = 1):
    """(page_table [B][max_pages] int32, number of physical pages); room for ``steps`` paths."""
    ps = w.page_size
    room = steps * (w.K + 1)
    need = [(int(L) + room + ps - 1) // ps for L in lens]
    max_pages = (w.max_prefix() + room + ps - 1) // ps
    total = int(sum(need))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TID_PAGES])))
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((w.B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total


def _cache(w: Workload, seed: int, tid: int, lens: np.ndarray, std: float, bf16: bool, table, steps: int = 1):
    """Prefix KV cache: contiguous [B][cap][H][Dh] or paged pool [P][page][H][Dh]."""
    row = w.H * w.Dh
    total = int(lens.sum())
    vals = normal_stream(seed, tid, total * row, std, bf16).reshape(total, row)
    dt = vals.dtype
    if not w.paged:
        cap = w.cache_capacity(steps)
        out = np.zeros((w.B, cap, w.H, w.Dh), dtype=dt)
        off = 0
        for b, L in enumerate(lens):
            out[b, :L] = vals[off:off + L].reshape(L, w.H, w.Dh)
            off += L
        return out
    ps = w.page_size
    npages = int(table.max()) + 1
    out = np.zeros((npages, ps, w.H, w.Dh), dtype=dt)
    off = 0
    for b, L in enumerate(lens):
        L = int(L)
        slots = np.arange(L)
        pages = table[b, slots // ps]
        out[pages, slots % ps] = vals[off:off + L].reshape(L, w.H, w.Dh)
        off += L
    return out


ALL_PARTS = ("h", "W1", "W2", "Wlm", "kv", "qkv")


def make_inputs(w: Workload, seed: int, parts=ALL_PARTS, steps: int = 1) -> dict:
    """Draw the inputs of one step (with ``steps`` > 1: of the first of that many chained steps).

    Returns a dict with (depending on ``parts``): ``h`` [B][d], ``W1`` [K][d][d],
    ``W2`` [K][V][d], ``Wlm`` [V][d], ``Kc``/``Vc`` (cache), ``q``/``k``/``v``
    [B][T][H][Dh], ``prefix_len`` [B] int32, ``page_table`` (paged only).
    bf16 tensors are uint16 bit patterns; fp32 tensors are float32.  ``steps``
    only sizes the cache: room for one accepted path (K+1 slots) per step.  The
    values drawn do not depend on it, except for a paged cache's page table.
    """
    bf16 = w.dtype == "bf16"
    std = float(w.d) ** -0.25
    T = w.n_nodes
    out = {"seed": seed, "workload": w.name}
    lens = prefix_lengths(w, seed)
    out["prefix_len"] = lens
    table = None
    if w.paged:
        table, _ = page_layout(w, seed, lens, steps)
        out["page_table"] = table
    if "h" in parts:
        out["h"] = normal_stream(seed, TID_H, w.B * w.d, std, bf16).reshape(w.B, w.d)
    if "W1" in parts:
        out["W1"] = normal_stream(seed, TID_W1, w.K * w.d * w.d, std, bf16).reshape(w.K, w.d, w.d)
    if "W2" in parts:
        out["W2"] = normal_stream(seed, TID_W2, w.K * w.V * w.d, std, bf16).reshape(w.K, w.V, w.d)
    if "Wlm" in parts:
        out["Wlm"] = normal_stream(seed, TID_WLM, w.V * w.d, std, bf16).reshape(w.V, w.d)
    if "kv" in parts:
        out["Kc"] = _cache(w, seed, TID_KC, lens, std, bf16, table, steps)
        out["Vc"] = _cache(w, seed, TID_VC, lens, std, bf16, table, steps)
    if "qkv" in parts:
        n = w.B * T * w.H * w.Dh
        shp = (w.B, T, w.H, w.Dh)
        out["q"] = normal_stream(seed, TID_Q, n, std, bf16).reshape(shp)
        out["k"] = normal_stream(seed, TID_K, n, std, bf16).reshape(shp)
        out["v"] = normal_stream(seed, TID_V, n, std, bf16).reshape(shp)
    return out


TID_STEP_QKV = 16  # tensor ids 16, 17, 18 (q, k, v) of step 1; +3 per further step


def step_qkv(w: Workload, seed: int, s: int) -> dict:
    """The tree's q/k/v inputs of step ``s`` of a chain (step 0: those of ``make_inputs``).

    In a full model they would come from the candidate tokens through the layers; here,
    as for the first step, they are independent seeded draws with the same recipe.
    """
    if s == 0:
        out = make_inputs(w, seed, parts=("qkv",))
        return {k: out[k] for k in ("q", "k", "v")}
    bf16 = w.dtype == "bf16"
    std = float(w.d) ** -0.25
    T = w.n_nodes
    n = w.B * T * w.H * w.Dh
    shp = (w.B, T, w.H, w.Dh)
    base = TID_STEP_QKV + 3 * (s - 1)
    return {name: normal_stream(seed, base + i, n, std, bf16).reshape(shp) for i, name in enumerate(("q", "k", "v"))}


TID_UNIFORM = 40  # + step index


def uniforms(w: Workload, seed: int, s: int = 0) -> dict:
    """Uniform random numbers in [0, 1) (float32) for rejection-sampling acceptance of step
    ``s``: ``u_accept`` [B][T] (one per tree node) and ``u_resample`` [B]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TID_UNIFORM + s])))
    T = w.n_nodes
    return {"u_accept": rng.random((w.B, T), dtype=np.float32),
            "u_resample": rng.random(w.B, dtype=np.float32)}


# ----------------------------------------------------------------------------
# full verify forward: decoder-layer weights and per-layer caches
# ----------------------------------------------------------------------------

TID_EMBED, TID_GFINAL = 900, 901
TID_LAYER = 1000  # + 16 * layer + j
LAYER_TENSORS = ("g_attn", "Wq", "Wk", "Wv", "Wo", "g_mlp", "Wg", "Wu", "Wd", "Kc", "Vc")


def _gain(seed: int, tid: int, n: int) -> np.ndarray:
    """Norm gains 1 + N(0, 0.1^2) as bf16 patterns."""
    z = normal_stream(seed, tid, n, 0.1, False)
    return f32_to_bf16_bits(z + np.float32(1.0))


def forward_inputs(dw, seed: int) -> dict:
    """The tensors the full forward adds to a step: ``E`` [V][d] (N(0, 1)) and ``g_final`` [d]."""
    w = dw.base
    return {"E": normal_stream(seed, TID_EMBED, w.V * w.d, 1.0, True).reshape(w.V, w.d),
            "g_final": _gain(seed, TID_GFINAL, w.d)}


def layer_inputs(dw, seed: int, layer: int, steps: int = 1) -> dict:
    """Layer ``layer``'s weights (bf16 patterns, [out][in]) and its prefix cache.

    Projection weights are N(0, 1/fan_in) so that each product keeps unit scale; gains
    are 1 + N(0, 0.1^2); the cache holds N(0, 1) keys/values (the scale of the tree's
    own keys and values) below each prefix length, zeros elsewhere.
    """
    w = dw.base
    d, F = w.d, dw.ffn
    tid = {n: TID_LAYER + 16 * layer + j for j, n in enumerate(LAYER_TENSORS)}
    sd, sf = float(d) ** -0.5, float(F) ** -0.5
    out = {"g_attn": _gain(seed, tid["g_attn"], d), "g_mlp": _gain(seed, tid["g_mlp"], d)}
    for n in ("Wq", "Wk", "Wv", "Wo"):
        out[n] = normal_stream(seed, tid[n], d * d, sd, True).reshape(d, d)
    out["Wg"] = normal_stream(seed, tid["Wg"], F * d, sd, True).reshape(F, d)
    out["Wu"] = normal_stream(seed, tid["Wu"], F * d, sd, True).reshape(F, d)
    out["Wd"] = normal_stream(seed, tid["Wd"], d * F, sf, True).reshape(d, F)
    lens = prefix_lengths(w, seed)
    table = page_layout(w, seed, lens, steps)[0] if w.paged else None
    out["Kc"] = _cache(w, seed, tid["Kc"], lens, 1.0, True, table, steps)
    out["Vc"] = _cache(w, seed, tid["Vc"], lens, 1.0, True, table, steps)
    return out
