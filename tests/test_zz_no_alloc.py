"""mdt_medusa_heads_noalloc (no workspace, nothing allocated) against mdt_medusa_heads.

Two calls in a row on the library's fixed device array, the second with a smaller
input (so it runs over the first call's leftovers): each must equal the workspace
call bit for bit (the same kernels, launched the same way), and the oracle's head
logits within the floating-point bar.
"""

import numpy as np
import pytest
import torch

from oracle import step as ostep
from tests.parity_util import REL_TOL, note, rel_err_rows
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _draw(rng, shape, std, bf16):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return f32_to_bf16_bits(x) if bf16 else x


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


# (dtype, B, d, V, K): batch 4 takes the matrix-core path, batch 1 the streaming GEMV; the
# largest case takes a third of the fixed array (16 * 5 * 4096 * 4 bytes of 4 MiB)
CALLS = [("bf16", 16, 4096, 1500, 5), ("bf16", 4, 512, 3001, 4), ("bf16", 1, 256, 2048, 3), ("f32", 2, 64, 512, 2)]


def test_noalloc_heads_match_workspace_call():
    import medusa_tree_verification_heads_amd as mdt
    for i, (dt, B, d, V, K) in enumerate(CALLS):
        note(f"noalloc heads call {i}: {dt} B={B} d={d} V={V} K={K}")
        rng = np.random.default_rng(100 + i)
        bf16 = dt == "bf16"
        std = d ** -0.25
        h = _draw(rng, (B, d), std, bf16)
        W1 = _draw(rng, (K, d, d), std, bf16)
        W2 = _draw(rng, (K, V, d), std, bf16)
        Wlm = _draw(rng, (V, d), std, bf16)
        hd, W1d, W2d, Wlmd = (_dev(a) for a in (h, W1, W2, Wlm))
        ref = mdt.medusa_heads(hd, W1d, W2d, Wlmd)
        got = torch.full((B, K + 1, V), float("nan"), device="cuda")
        mdt.medusa_heads_noalloc(hd, W1d, W2d, Wlmd, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i
        if B * d * V <= 4 * 512 * 3001:
            logits, _ = ostep.medusa_heads(h, W1, W2, Wlm)
            assert rel_err_rows(got.cpu().numpy(), logits) <= REL_TOL, i

