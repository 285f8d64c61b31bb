"""The five workloads of the Medusa draft-and-verify step, plus scaled-down variants.

Shapes follow the Vicuna model sizes named on the Medusa pages ("Medusa: Simple
LLM Inference Acceleration Framework with Multiple Decoding Heads", section
"MEDUSA Heads: Architecture and Mechanism": d = 4096 and V = 32,000 for the 7B
backbone, at most five heads) and the 64-node sparse tree of section "Optimized
Tree Construction".  Trained weights, MT-Bench prompts and the calibration set
are not available, so every tensor is synthetic (see ``gen.py``) and the
per-node accuracy of the sparse tree is the synthetic rule
``a0 * rho**rank * gamma**(head-1)`` (rank 0-based, head 1..K).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class AcceptRun:
    mode: str            # "greedy" or "typical"
    temperature: float   # tau; 0 means greedy verifier distribution
    eps: float = 0.09
    delta: float = 0.3


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": storage type of weights, h, KV, q/k/v
    B: int                     # sequences per step
    d: int                     # hidden size (= H * Dh)
    H: int                     # attention heads
    Dh: int                    # head dim
    V: int                     # vocabulary
    K: int                     # Medusa heads (the LM head is extra)
    k_cfg: int                 # top-k computed for every head row
    tree_kind: str             # "cartesian" or "scored"
    tree_s: Tuple[int, ...] = ()   # cartesian: candidates per depth (s_1..s_K)
    T: int = 0                 # scored: nodes including the root
    a0: float = 0.6
    rho: float = 0.7
    gamma: float = 0.8
    L: int = 0                 # prefix length (contiguous KV); ignored when L_range is set
    L_range: Optional[Tuple[int, int]] = None   # inclusive uniform range of per-sequence prefix lengths
    paged: bool = False
    page_size: int = 16
    rope_theta: float = 10000.0
    accept: Tuple[AcceptRun, ...] = field(default_factory=tuple)

    @property
    def n_nodes(self) -> int:
        if self.tree_kind == "cartesian":
            tot, prod = 1, 1
            for s in self.tree_s:
                prod *= s
                tot += prod
            return tot
        return self.T

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def max_prefix(self) -> int:
        return self.L_range[1] if self.L_range else self.L

    def cache_capacity(self, steps: int = 1) -> int:
        """Slots per sequence: the prefix plus room for one accepted path (K+1 tokens) per step."""
        return self.max_prefix() + steps * (self.K + 1)


TYPICAL_07 = AcceptRun("typical", 0.7, 0.09, 0.3)
GREEDY = AcceptRun("greedy", 0.0)

WORKLOADS = {
    # Tiny reference step, fp32: top-(3,2) Cartesian tree, T = 1 + 3 + 6 = 10.
    "tiny-fp32-T10": Workload(
        name="tiny-fp32-T10", dtype="f32", B=1, d=64, H=4, Dh=16, V=512, K=2, k_cfg=3,
        tree_kind="cartesian", tree_s=(3, 2), L=32,
        accept=(GREEDY, AcceptRun("typical", 0.0, 0.09, 0.3))),
    # Vicuna-7B-shaped layer, 64-node sparse tree, prefix 1024, batch 1.
    "7b-T64-L1024": Workload(
        name="7b-T64-L1024", dtype="bf16", B=1, d=4096, H=32, Dh=128, V=32000, K=4, k_cfg=10,
        tree_kind="scored", T=64, L=1024, accept=(GREEDY, TYPICAL_07)),
    # Vicuna-13B-shaped layer, 64-node sparse tree, prefix 4096, batch 1, typical at tau 0.7.
    "13b-T64-L4096": Workload(
        name="13b-T64-L4096", dtype="bf16", B=1, d=5120, H=40, Dh=128, V=32000, K=5, k_cfg=10,
        tree_kind="scored", T=64, L=4096, accept=(TYPICAL_07, AcceptRun("typical", 0.0, 0.09, 0.3))),
    # Batched 7B-shaped step, 42-node tree per sequence, batch 16, paged KV (16-token pages).
    "7b-B16-T42-paged": Workload(
        name="7b-B16-T42-paged", dtype="bf16", B=16, d=4096, H=32, Dh=128, V=32000, K=4, k_cfg=10,
        tree_kind="scored", T=42, L_range=(512, 8192), paged=True, page_size=16,
        accept=(GREEDY, TYPICAL_07)),
    # Vicuna-33B-shaped layer, 256-node tree, prefix 16384, batch 4.
    "33b-B4-T256-L16384": Workload(
        name="33b-B4-T256-L16384", dtype="bf16", B=4, d=6656, H=52, Dh=128, V=32000, K=5, k_cfg=16,
        tree_kind="scored", T=256, L=16384, accept=(GREEDY, TYPICAL_07)),
}

# The workload the headline throughput is quoted on.
HEADLINE = "7b-T64-L1024"


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced-size parity cases)."""
    if "name" not in changes:
        tag = ",".join(f"{k}={v}" for k, v in sorted(changes.items()))
        changes["name"] = f"{w.name}[{tag}]"
    return dataclasses.replace(w, **changes)


# Reduced-size cases for element-by-element parity: same structure as the five
# workloads, sizes the oracle finishes in seconds, spanning several kernel tiles
# with ragged tails (V, L not multiples of any tile).
PARITY_CASES = {
    "tiny-fp32-T10": WORKLOADS["tiny-fp32-T10"],
    "7b-mini": scaled(WORKLOADS["7b-T64-L1024"], name="7b-mini", d=512, H=4, V=3001, L=300),
    "13b-mini": scaled(WORKLOADS["13b-T64-L4096"], name="13b-mini", d=640, H=5, V=2500, L=517),
    "7b-B16-mini-paged": scaled(WORKLOADS["7b-B16-T42-paged"], name="7b-B16-mini-paged", B=4, d=512, H=4,
                                V=3001, L_range=(17, 200)),
    "33b-mini": scaled(WORKLOADS["33b-B4-T256-L16384"], name="33b-mini", B=2, d=384, H=3, V=2048, L=700),
}


def get_case(name: str) -> Workload:
    return PARITY_CASES[name] if name in PARITY_CASES else WORKLOADS[name]


# ----------------------------------------------------------------------------
# Full verify forward: the tree through a stack of decoder layers
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class DeepWorkload:
    """A step workload whose tree goes through ``n_layers`` synthetic Llama decoder layers
    (RMSNorm, q/k/v, tree attention, output projection, RMSNorm, SwiGLU feed-forward of
    width ``ffn``) and a final RMSNorm before the LM head.  Vicuna-7B has 32 layers of
    feed-forward width 11008."""
    name: str
    base: Workload
    n_layers: int
    ffn: int
    norm_eps: float = 1e-6


FORWARD_WORKLOADS = {
    "7b-T64-L1024-x32": DeepWorkload("7b-T64-L1024-x32", WORKLOADS["7b-T64-L1024"], 32, 11008),
}

# Parity cases of the forward: the 7B mini with two layers (also with two sequences), and
# two layers at full 7B width.
FORWARD_CASES = {
    "7b-mini-x2": DeepWorkload("7b-mini-x2", PARITY_CASES["7b-mini"], 2, 1376),
    "7b-mini-B2-x2": DeepWorkload("7b-mini-B2-x2", scaled(PARITY_CASES["7b-mini"], name="7b-mini-B2", B=2), 2, 1376),
    "7b-T64-L1024-x2": DeepWorkload("7b-T64-L1024-x2", WORKLOADS["7b-T64-L1024"], 2, 11008),
}
