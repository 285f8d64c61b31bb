"""Seed search for bit-exact parity cases (run offline; writes ``workloads/seeds.json``).

For each workload (the five full-size ones and the reduced parity cases) try
seeds ``1000 * index + attempt`` and keep the first whose oracle step takes every
discrete decision with margin >= ``margins.MIN_MARGIN`` in every acceptance
run of the workload.  Only this package (``oracle``) and the input generator are
used.

    python -m oracle.find_seeds [name ...]
"""

from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

from workloads import make_inputs
from workloads.configs import PARITY_CASES, WORKLOADS

from . import margins, step, tree as otree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "workloads", "seeds.json")

ORDER = list(WORKLOADS) + [n for n in PARITY_CASES if n not in WORKLOADS]


def case_margin(w, seed: int) -> float:
    inp = make_inputs(w, seed)
    tree = otree.build_tree(w)
    logits, _ = step.medusa_heads(inp["h"], inp["W1"], inp["W2"], inp["Wlm"])
    m = margins.head_margin(logits, w.k_cfg)
    K1 = w.K + 1
    tk = np.empty((w.B, K1, w.k_cfg), dtype=np.int64)
    for b in range(w.B):
        for r in range(K1):
            tk[b, r] = step.topk(logits[b, r], w.k_cfg)[0]
    tokens, _ = step.tree_expand(tk, tree, inp["prefix_len"])
    o, _ = step.tree_attention(inp["q"], inp["k"], inp["v"], inp["Kc"], inp["Vc"], inp["prefix_len"], tree,
                               w.rope_theta, bf16_store=(w.dtype == "bf16"), page_table=inp.get("page_table"),
                               page_size=w.page_size)
    x = o.reshape(w.B * tree.T, w.d)
    del inp
    z, _ = step.verify_logits(x, make_inputs(w, seed, parts=("Wlm",))["Wlm"], 0.0)
    for run in w.accept:
        stats = [step.row_stats(z[r], run.temperature) for r in range(z.shape[0])]
        e = margins.edge_margins(z, stats, tokens, tree, run.mode, run.eps, run.delta, run.temperature)
        m = min(m, float(e.min()))
    return m


def main(names):
    seeds = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        idx = ORDER.index(name) + 1
        w = PARITY_CASES.get(name) or WORKLOADS[name]
        for attempt in range(100):
            seed = 1000 * idx + attempt
            t0 = time.time()
            m = case_margin(w, seed)
            print(f"{name} seed {seed}: margin {m:.3e} ({time.time() - t0:.1f}s)", flush=True)
            if m >= margins.MIN_MARGIN:
                seeds[name] = {"seed": seed, "margin": m}
                break
        else:
            raise SystemExit(f"no seed found for {name}")
        json.dump(seeds, open(OUT, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ORDER)
