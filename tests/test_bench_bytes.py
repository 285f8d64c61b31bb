"""The byte counts behind bench.py's HBM figures, against the method's own sizes (CPU only).

At the 7B-shaped step every weight is read once per use: W1 (K d^2), W2 (K d V) and W_lm
twice (the LM head on h, the verifier on the tree rows), plus the prefix keys and values
once; the tree tensors, logits and other small reads and writes add under 0.3 %.  The dominant kernel's per-launch figure is
W2 plus its own small reads and writes.  The full forward adds every decoder layer's
weights (q, k, v, output: 4 d^2; gate, up, down: 3 d F; two norm gains) and prefix cache.
"""

import bench
from workloads.configs import FORWARD_WORKLOADS, get_case


def test_step_bytes_at_the_headline():
    w = get_case("7b-T64-L1024")
    T = 64
    ab = bench.algorithmic_bytes(w, T, [1024])
    d, V, K, e = w.d, w.V, w.K, 2
    weights = e * (K * d * d + K * d * V + 2 * d * V)
    kv = e * 2 * 1024 * w.H * w.Dh
    assert weights == 134_217_728 + 1_048_576_000 + 2 * 262_144_000   # W1 + W2 + 2 W_lm
    assert ab["total"] > weights + kv
    assert (ab["total"] - weights - kv) / ab["total"] < 3e-3
    assert ab["total"] == 1_728_587_776
    # the dominant launch: W2 once, plus a (fp32 in) and its logits (fp32 out)
    assert ab["heads_gemv_w2"] == e * K * V * d + 4 * K * d + 4 * K * V


def test_forward_bytes_at_32_layers():
    dw = FORWARD_WORKLOADS["7b-T64-L1024-x32"]
    w = dw.base
    fb = bench.forward_bytes(dw, 64, [1024])
    d, F, nL = w.d, dw.ffn, dw.n_layers
    assert fb["layer_weights"] == nL * 2 * (4 * d * d + 3 * d * F + 2 * d)
    assert fb["prefix_kv"] == nL * 2 * 2 * 1024 * w.H * w.Dh
    step = bench.algorithmic_bytes(w, 64, [1024])["total"]
    assert fb["total"] > fb["layer_weights"] + fb["prefix_kv"] + step - 2 * 2 * 64 * 5 * d
    assert fb["total"] == 15_546_034_176
