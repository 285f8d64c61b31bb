"""The heads of batches on the matrix cores (B >= 4, bf16): logits against the oracle.

Batch sizes cover every tile shape the path launches (B <= 8: one 16-row m-tile in
both launches; B <= 16: two in the second; B <= 32: two and four), plus B = 3 (the
GEMV path) for contrast.  a = SiLU(W1 h) + h is carried into the second product as two
bf16 halves (about 16 significant bits), so the logits stay within 1e-4 of each row's
largest magnitude (the bf16 GEMV path is within about 1e-6); the top-k decisions of the
parity tests need margins of 1e-3.
"""

import numpy as np
import pytest
import torch

from oracle import step as ostep
from tests.parity_util import note
from workloads import make_inputs
from workloads.configs import PARITY_CASES, scaled

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,d", [(3, 512), (4, 512), (7, 512), (12, 512), (17, 512), (32, 512), (5, 576),
                                 (20, 576)])
def test_heads_batch_matches_oracle(B, d):
    """d = 512: the DMA-staged tiles (d a multiple of 128); d = 576: the register-staged ones."""
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.step import to_device
    w = scaled(PARITY_CASES["7b-mini"], name=f"7b-mini-B{B}-d{d}", B=B, d=d)
    inp = make_inputs(w, 4242 + B + d, parts=("h", "W1", "W2", "Wlm"))
    t = {k: to_device(inp[k], "cuda") for k in ("h", "W1", "W2", "Wlm")}
    logits = mdt.medusa_heads(t["h"], t["W1"], t["W2"], t["Wlm"])
    torch.cuda.synchronize()
    g = logits.cpu().numpy().astype(np.float64)
    ref, _ = ostep.medusa_heads(inp["h"], inp["W1"], inp["W2"], inp["Wlm"])
    err = np.abs(g - ref).max(axis=2) / np.abs(ref).max(axis=2)
    note(f"heads B={B} d={d}: max rel err {err.max():.2e}")
    assert err.max() <= 1e-4


@pytest.mark.parametrize("B", [1, 2, 8])
def test_heads_without_lm_head(B):
    """Wlm = NULL: slot 0 keeps what it held, slots 1..K are bit for bit those of the full call
    (the vector-ALU path below four sequences, the matrix-core path from four on)."""
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.step import to_device
    w = scaled(PARITY_CASES["7b-mini"], name=f"7b-mini-B{B}", B=B)
    inp = make_inputs(w, 5151 + B, parts=("h", "W1", "W2", "Wlm"))
    t = {k: to_device(inp[k], "cuda") for k in ("h", "W1", "W2", "Wlm")}
    full = mdt.medusa_heads(t["h"], t["W1"], t["W2"], t["Wlm"])
    part = torch.full_like(full, 7.5)
    mdt.medusa_heads(t["h"], t["W1"], t["W2"], None, logits=part)
    torch.cuda.synchronize()
    assert torch.all(part[:, 0] == 7.5)
    assert torch.equal(part[:, 1:], full[:, 1:])
