"""Whole-step GPU properties: repeated calls give identical bits (every reduction and
merge runs in a fixed order, independent of workgroup scheduling), and a HIP-graph
capture of the step replays to the eager result."""

import numpy as np
import pytest
import torch

from tests.parity_util import case_inputs, note

pytestmark = pytest.mark.gpu

KEYS = ("logits", "topk_idx", "tokens", "pos", "o", "k_rot", "stats", "edge", "path", "n_acc", "new_len", "Kc", "Vc")


def _make(name, run_idx=1, fused_tail=True, tail="verify_accept_compact", want_logits=False):
    from medusa_tree_verification_heads_amd.step import VerifyStep
    w, inp = case_inputs(name)
    run = w.accept[min(run_idx, len(w.accept) - 1)]
    note(f"step {name} {run} fused_tail={fused_tail} tail={tail}")
    return VerifyStep(w, inp, run.mode, run.temperature, run.eps, run.delta, fused_tail=fused_tail, tail=tail,
                      want_logits=want_logits)


def _same(a, b):
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["7b-mini", "7b-B16-mini-paged", "33b-mini", "tiny-fp32-T10"])
def test_repeated_steps_are_bit_identical(name):
    s = _make(name)
    s.run()
    first = s.outputs()
    for _ in range(3):
        s.run()
        _same(first, s.outputs())


@pytest.mark.parametrize("run_idx", [0, 1])
@pytest.mark.parametrize("name", ["7b-mini", "7b-B16-mini-paged", "33b-mini", "tiny-fp32-T10"])
def test_fused_tail_matches_separate_calls(name, run_idx):
    """verify_accept_compact writes exactly what verify_logits, accept_path and kv_compact
    write, and so does verify_logits then accept_compact (full logits included)."""
    sep = _make(name, run_idx, fused_tail=False, want_logits=True)
    sep.run()
    ref = sep.outputs()
    for tail in ("accept_compact", "verify_accept_compact"):
        fused = _make(name, run_idx, tail=tail, want_logits=True)
        fused.run()
        out = fused.outputs()
        _same(ref, out)
        assert np.array_equal(ref["vlogits"], out["vlogits"])


@pytest.mark.parametrize("name", ["7b-mini", "7b-B16-mini-paged"])
def test_graph_replay_matches_eager(name):
    s = _make(name)
    s.run()
    eager = s.outputs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        s.run()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        _same(eager, s.outputs())
        s.run()           # eager work between replays
        torch.cuda.synchronize()
        _same(eager, s.outputs())
