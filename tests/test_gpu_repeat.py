"""Repeated calls reproduce every output bit for bit.

Every kernel of the step reduces in a fixed order (no atomics, no result that depends on
which workgroup finishes first), and the compaction writes the same rows past the same
prefix on every call, so running the step again on the same inputs must reproduce every
output exactly: head logits, top-k, tree tokens and positions, the attention output and
rotated keys, row statistics and edge logits, the accepted path and lengths, and the
whole cache.  A mismatch here is a race (a read that some launch order can reach before
its write), which value tolerances against the oracle could let through.

Cases: every reduced parity case, and the full-size workloads whose launches differ most
(the batch-1 GEMV heads and 64-row verifier of the 7B headline, the matrix-core heads,
wide verifier tiles and paged attention of the 16-sequence batch, the 256-node trees with
two query tiles per wave of the 33B shape).  The headline step is also captured as one
HIP graph and replayed several times, with eager work between the replays, every replay
checked against the eager step.
"""

import numpy as np
import pytest
import torch

from tests.parity_util import SEEDS, note
from workloads import make_inputs
from workloads.configs import PARITY_CASES, WORKLOADS

pytestmark = pytest.mark.gpu

FULL = ["7b-T64-L1024", "7b-B16-T42-paged", "33b-B4-T256-L16384"]


def _seed(name):
    if name in SEEDS:
        return SEEDS[name]["seed"]
    return 1000 * (list(WORKLOADS).index(name) + 1)


def _snapshot(s) -> dict:
    """Device copies of every output of VerifyStep s."""
    out = dict(logits=s.logits, topk_idx=s.topk_idx, topk_val=s.topk_val, tokens=s.tokens, pos=s.pos, o=s.o,
               k_rot=s.k_rot, stats=s.stats, edge=s.edge, path=s.path, n_acc=s.n_acc, new_len=s.new_len,
               Kc=s.t["Kc"], Vc=s.t["Vc"])
    return {k: v.detach().clone() for k, v in out.items()}


def _assert_same_bits(a: dict, b: dict, what: str):
    for k in a:
        x, y = a[k].contiguous().view(torch.uint8), b[k].contiguous().view(torch.uint8)
        if not torch.equal(x, y):
            diff = int((x != y).sum())
            raise AssertionError(f"{what}: output {k} differs in {diff} of {x.numel()} bytes")


def _step(name, w):
    from medusa_tree_verification_heads_amd.step import VerifyStep
    inp = make_inputs(w, _seed(name))
    run = w.accept[-1]
    note(f"repeat {name} seed {_seed(name)} run {run}")
    return VerifyStep(w, inp, run.mode, run.temperature, run.eps, run.delta)


@pytest.mark.parametrize("name", list(PARITY_CASES))
def test_repeat_reduced(name):
    s = _step(name, PARITY_CASES[name])
    s.run()
    first = _snapshot(s)
    for i in range(2):
        s.run()
        torch.cuda.synchronize()
        _assert_same_bits(first, _snapshot(s), f"{name} call {i + 2}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", FULL)
def test_repeat_full(name):
    s = _step(name, WORKLOADS[name])
    s.run()
    first = _snapshot(s)
    s.run()
    torch.cuda.synchronize()
    _assert_same_bits(first, _snapshot(s), f"{name} call 2")


@pytest.mark.timeout(300)
def test_repeat_graph_replays():
    name = "7b-T64-L1024"
    s = _step(name, WORKLOADS[name])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = _snapshot(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.run()
    scratch = torch.zeros(1 << 20, device="cuda")
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        _assert_same_bits(eager, _snapshot(s), f"{name} graph replay {i + 1}")
        scratch.add_(1.0)   # the program's own eager work between replays
        s.logits.zero_()    # outputs cleared, so a replay that skipped a kernel would show
        s.o.zero_()
        torch.cuda.synchronize()
    assert float(scratch[0]) == 3.0
