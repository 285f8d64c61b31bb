#!/usr/bin/env python3
"""Throughput of the Medusa draft-and-verify step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload 7b-T64-L1024] [--mode typical]

A step is one pass of the whole path -- medusa_heads, topk_tree_expand,
tree_attention, verify_logits, accept_path, kv_compact -- over one batch of
synthetic inputs already resident in HBM.  W untimed warm-up steps run first.
A profiled pass of K eager steps then launches every kernel with start/stop HIP
events on its own stream (hipExtLaunchKernelGGL), giving each kernel's duration;
the roofline object uses the dominant kernel's (the W2 head GEMV stream).  The
timed region is K replays of a HIP graph that holds the whole step (warmed by at
least GRAPH_WARMUP untimed replays: a fresh graph's first replays are slower), between two
torch.cuda.synchronize() calls (the events add dispatch gaps, so they stay out
of it); afterwards K more replays, each between two events, give the median, p10
and p90 per step (``replay_us``), and a 1 GiB device copy gives the copy bandwidth
that ``step_hbm.frac_of_copy`` divides by.  The CPU oracle is timed on the host on whole steps of the same
workload (its one-time bf16 -> float64 upcast reported apart, then the median of 3 steps with all
BLAS threads and of 3 with one).  A report of chained steps (``decode_loop``: each step
starts from the previous step's last accepted node, replayed as one graph) gives
the time per chained step and the synthetic acceptance; a report of the full
verify forward (``full_depth``: the tree through all 32 decoder layers of the
7B-shaped model before the LM head, one graph) gives its time per step and HBM
fraction.  Both are context, not the metric.  One JSON line goes to stdout.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X published HBM3E bandwidth
LOOP_STEPS = 8           # chained steps of the decode-loop report
GRAPH_WARMUP = 60        # untimed replays of the captured step before the timed region
METRIC = "Medusa verify-steps/s + achieved HBM GB/s vs peak, 7B-shape 64-node tree"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, T, lens):
    """Bytes the step must move (each weight once per use, prefix KV once, tree tensors once)."""
    e = w.elt_bytes
    B, d, V, K, H, Dh = w.B, w.d, w.V, w.K, w.H, w.Dh
    heads_w1_lm = e * (K * d * d + d * V) + B * e * d + B * 4 * (K * d + V)
    heads_w2 = e * K * V * d + B * 4 * K * d + B * 4 * K * V
    topk = B * 4 * (K + 1) * V
    attn = e * 2 * int(sum(int(x) for x in lens)) * H * Dh + e * B * T * 5 * d
    verify = e * V * d + e * B * T * d
    compact = 2 * 2 * e * B * (K + 1) * d
    total = heads_w1_lm + heads_w2 + topk + attn + verify + compact
    return dict(heads_gemv_w1_lm=heads_w1_lm, heads_gemv_w2=heads_w2, topk=topk, attention=attn,
                verify_mfma=verify, compact=compact, total=total)


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "medusa_tree_verification_heads_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(f"{kernel}@{workload}")
    if not rec or rec.get("src_digest") != digest:
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(w, inp, mode, tau, eps, delta, nsteps=3):
    """The oracle as it stands, timed on whole steps on the host cores: the one-time upcast of
    the bf16 inputs to float64 is timed and reported on its own, then the median of nsteps
    steps on the float64 inputs with every BLAS thread, then the median of nsteps on one."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import step as ostep
    from oracle import tree as otree
    tree = otree.build_tree(w)
    t0 = time.perf_counter()
    inp64 = {k: (ostep.to_f64(v) if isinstance(v, np.ndarray) and v.dtype == np.uint16 else v)
             for k, v in inp.items()}
    upcast_s = time.perf_counter() - t0

    def median_step():
        ts = []
        for _ in range(nsteps):
            t = time.perf_counter()
            ostep.step(w, inp64, tree, mode, tau, eps, delta)
            ts.append(time.perf_counter() - t)
        return float(np.median(ts)), ts

    med, ts = median_step()
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    with threadpool_limits(limits=1):
        med1, ts1 = median_step()
    model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                 platform.processor() or "cpu") if os.path.exists("/proc/cpuinfo") else platform.processor()
    return {"value": round(1.0 / med, 6), "unit": "verify-steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"median of {nsteps} full oracle steps of {w.name} (all six stages, float64 NumPy) on "
                      f"inputs already upcast to float64 in host memory (steps {', '.join(f'{t:.2f}' for t in ts)} s); "
                      f"host {model}, {len(os.sched_getaffinity(0))} affinity cores of {os.cpu_count()}",
            "upcast_s": round(upcast_s, 3),
            "single_core": {"value": round(1.0 / med1, 6), "cores": 1,
                            "sample": f"median of {nsteps} steps with one BLAS thread "
                                      f"({', '.join(f'{t:.2f}' for t in ts1)} s)"}}


def decode_loop_report(w, inp, seed, step, mode, tau, eps, delta, replays):
    """LOOP_STEPS chained steps (the next step starts from the last accepted node), replayed as
    one HIP graph: time per chained step and the synthetic acceptance (tokens per step)."""
    import numpy as np
    import torch
    from medusa_tree_verification_heads_amd.step import DecodeLoop
    from workloads import step_qkv
    qkv = [step_qkv(w, seed, s) for s in range(LOOP_STEPS)]
    loop = DecodeLoop(w, inp, qkv, mode, tau, eps, delta, step=step)
    loop.run()
    torch.cuda.synchronize()
    n_acc = loop.n_acc.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        loop.run()
    reps = max(1, replays // LOOP_STEPS)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / (reps * LOOP_STEPS)
    mean_acc = float(n_acc.mean())
    return {"steps": LOOP_STEPS, "us_per_step": round(us, 2), "mean_accepted_per_step": round(mean_acc, 3),
            "accepted_tokens_per_s": round(1e6 / us * mean_acc * w.B, 1),
            "n_acc_per_step": n_acc[:, 0].tolist(),
            "lm_head": "steps after the first take the LM-head row from the verifier (next_logits)",
            "note": "synthetic random weights: the acceptance is not that of a trained model"}


def forward_bytes(dw, T, lens):
    """Bytes the full-forward step must move: the step's heads, top-k and LM-head bytes,
    every layer's weights once, every layer's prefix KV once, the embedding rows, and the
    layer activations (each written once and read once per use)."""
    w = dw.base
    ab = algorithmic_bytes(w, T, lens)
    e, B, d, F, M, nL = w.elt_bytes, w.B, w.d, dw.ffn, w.B * T, dw.n_layers
    layer_w = e * (3 * d * d + d * d + 2 * F * d + d * F + 2 * d)
    kv = e * 2 * int(sum(int(x) for x in lens)) * w.H * w.Dh
    # per layer: h (w+r), q|k|v (w+r), k_rot (w), o (w+r), x (r+w twice), a (w+r), fp32 slices (w+r)
    act = e * M * (2 * d + 6 * d + d + 2 * d + 4 * d + 2 * F)
    total = (ab["heads_gemv_w1_lm"] + ab["heads_gemv_w2"] + ab["topk"] + ab["verify_mfma"] + e * M * d
             + nL * (layer_w + kv + act + 2 * 2 * e * B * (w.K + 1) * d))
    return {"layer_weights": nL * layer_w, "prefix_kv": nL * kv, "total": total}


def full_depth_report(w, seed, step, mode, tau, eps, delta, replays):
    """The step with the full verify forward: the tree through every decoder layer of the
    7B-shaped model (32 layers, feed-forward 11008) before the LM head.  Layer weights,
    embedding and per-layer caches are drawn on the GPU with a seeded torch generator
    (13 GB); the heads and LM head are the step's own.  Replayed as one HIP graph."""
    import numpy as np
    import torch
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.forward import VerifyForward
    from workloads.configs import FORWARD_WORKLOADS
    dw = next((f for f in FORWARD_WORKLOADS.values() if f.base.name == w.name), None)
    if dw is None:
        return None
    dev = step.dev
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    d, F, nL = w.d, dw.ffn, dw.n_layers

    def rn(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    def gain():
        return (1 + torch.randn((d,), generator=gen, device=dev) * 0.1).to(torch.bfloat16)

    layers = [{"g_attn": gain(), "Wqkv": rn((3 * d, d), d ** -0.5), "Wo": rn((d, d), d ** -0.5), "g_mlp": gain(),
               "Wgu": rn((2 * F, d), d ** -0.5), "Wd": rn((d, F), F ** -0.5)} for _ in range(nL)]
    cap = w.cache_capacity(1)
    lens = step.prefix_len
    Kc = torch.zeros((nL, w.B, cap, w.H, w.Dh), dtype=torch.bfloat16, device=dev)
    Vc = torch.zeros_like(Kc)
    for b in range(w.B):
        L = int(lens[b])
        Kc[:, b, :L] = rn((nL, L, w.H, w.Dh), 1.0)
        Vc[:, b, :L] = rn((nL, L, w.H, w.Dh), 1.0)
    f = VerifyForward(dw, step.t, rn((w.V, d), 1.0), gain(), layers, Kc, Vc, lens, mode, tau, eps, delta,
                      tree=None)
    for _ in range(2):
        f.run()
    torch.cuda.synchronize()
    timer = mdt.KernelTimer(16 * nL + 16)
    with timer:
        f.run()
    torch.cuda.synchronize()
    per = {}
    for k, ms in timer.durations_ms():
        per[k] = per.get(k, 0.0) + 1e3 * ms
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        f.run()
    g.replay()
    torch.cuda.synchronize()
    reps = max(3, replays // 20)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / reps
    fb = forward_bytes(dw, f.tree.T, [int(x) for x in lens.cpu()])
    gbps = fb["total"] / (us * 1e-6) / 1e9
    lin = fb["layer_weights"] / (per.get("linear_mfma", 0) * 1e-6) / 1e9 if per.get("linear_mfma") else None
    rep = {"workload": dw.name, "layers": nL, "ffn": F, "us_per_step": round(us, 1),
           "steps_per_s": round(1e6 / us, 2), "tree_tokens_per_s": round(1e6 / us * f.M, 1),
           "algorithmic_bytes": fb["total"], "achieved_GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
           "linear_weight_GBps": round(lin, 1) if lin else None, "splits": [f.split_o, f.split_d],
           "per_kernel_us_per_step": {k: round(v, 1) for k, v in per.items()},
           "n_acc": f.n_acc.cpu().tolist()[:8],
           "weights": "drawn on the GPU with a seeded torch generator (13 GB), random: acceptance is not a "
                      "trained model's"}
    del f, layers, Kc, Vc
    torch.cuda.empty_cache()
    return rep


def copy_bandwidth(mib: int = 1024, reps: int = 5) -> float:
    """HBM bandwidth of a plain device-to-device copy of `mib` MiB (bytes read + written per
    second, best of `reps` copies timed with events); the buffers are freed afterwards."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / best / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--mode", default="typical", choices=["typical", "greedy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-loop", action="store_true", help="skip the chained-step (decode loop) report")
    ap.add_argument("--no-full-depth", action="store_true", help="skip the full verify forward report")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU layout is a design note, not a built path", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return

    if not os.path.exists(os.path.join(ROOT, "medusa_tree_verification_heads_amd", "libmdt.so")):
        from __graft_entry__ import _builder
        _builder().build()
    import numpy as np
    import torch
    import medusa_tree_verification_heads_amd as mdt
    from medusa_tree_verification_heads_amd.step import VerifyStep
    from workloads import make_inputs
    from workloads.configs import HEADLINE, get_case

    name = args.workload or HEADLINE
    w = get_case(name)
    seeds = json.load(open(os.path.join(ROOT, "workloads", "seeds.json")))
    seed = seeds.get(name, {"seed": 0})["seed"]
    run = next((r for r in w.accept if r.mode == args.mode), None)
    tau = run.temperature if run else (0.7 if args.mode == "typical" else 0.0)
    eps, delta = (run.eps, run.delta) if run else (0.09, 0.3)
    t0 = time.perf_counter()
    inp = make_inputs(w, seed, steps=LOOP_STEPS)   # cache room for the chained-step report
    log(f"inputs for {name} (seed {seed}) drawn in {time.perf_counter() - t0:.1f}s")
    step = VerifyStep(w, inp, args.mode, tau, eps, delta)
    T = step.tree.T
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log(f"warm-up done ({args.warmup} steps)")

    # per-kernel pass: K eager steps, every kernel launched with start/stop events on its stream
    per_step = 16   # >= kernels per step
    timer = mdt.KernelTimer(per_step * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with timer:
        for _ in range(args.steps):
            step.run()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per_kernel = {}
    for kname, ms in timer.durations_ms():
        per_kernel.setdefault(kname, []).append(ms)
    per_kernel_us = {k: round(1e3 * float(np.mean(v)), 2) for k, v in per_kernel.items()}
    log(f"profiled eager pass: {eager_ms * 1e3:.1f} us/step; kernels {per_kernel_us}")

    replay_us = None
    if args.no_graph:
        ms_per_step, timing = eager_ms, "eager launches with per-kernel events"
    else:
        # timed region: K replays of a HIP graph holding the whole step (no events inside)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step.run()
        # a freshly captured graph runs its first few dozen replays 3-4 % slower (measured:
        # 307, 304, then 297-296 us per step over consecutive batches of 20), a one-time
        # cost that is not part of a step: the graph is warmed with at least GRAPH_WARMUP
        # replays before the timed region
        for _ in range(max(args.warmup, GRAPH_WARMUP)):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps
        timing = "HIP-graph replay of the six calls"
        # distribution (outside the timed region): every replay between two events
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        replay_us = {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
                     "p90": round(float(np.percentile(us, 90)), 2), "replays": args.steps}
        log(f"per-replay us: {replay_us}")
    log(f"timed {args.steps} steps ({timing}): {ms_per_step * 1e3:.1f} us/step")
    copy_gbps = copy_bandwidth()

    loop_rep = None
    if not args.no_graph and not args.no_loop:
        loop_rep = decode_loop_report(w, inp, seed, step, args.mode, tau, eps, delta, args.steps)
        log(f"decode loop: {loop_rep}")

    full_rep = None
    if not args.no_graph and not args.no_full_depth:
        full_rep = full_depth_report(w, seed, step, args.mode, tau, eps, delta, args.steps)
        log(f"full verify forward: {full_rep}")

    lens = inp["prefix_len"]
    ab = algorithmic_bytes(w, T, lens)
    # the W2 head stream: the GEMV at B < 4, the matrix-core tile for larger batches
    dom = "heads_gemv_w2" if "heads_gemv_w2" in per_kernel_us else "heads_mfma_w2"
    dom_us = per_kernel_us.get(dom)
    achieved = ab["heads_gemv_w2"] / (dom_us * 1e-6) / 1e9 if dom_us else None
    digest = src_digest("heads.hip", "common.h")
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4) if achieved else None,
                "traffic": measured_traffic(dom, name, digest),
                "bytes_per_launch": ab["heads_gemv_w2"], "avg_launch_us": dom_us}
    step_gbps = ab["total"] / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 2),
        "unit": "verify-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "d": w.d, "H": w.H, "Dh": w.Dh, "V": w.V, "K": w.K,
                   "k_cfg": w.k_cfg, "T": T, "prefix": [int(x) for x in lens][:4] if w.B > 4 else
                   [int(x) for x in lens], "paged": w.paged, "accept": args.mode, "tau": tau, "eps": eps,
                   "delta": delta, "seed": seed, "parallelism": "none (1 GPU)"},
        "tree_tokens_per_s": round(1e3 / ms_per_step * w.B * T, 1),
        "step_hbm": {"algorithmic_bytes": ab["total"], "achieved": round(step_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(step_gbps / PEAK_HBM_GBPS, 4),
                     "copy_GBps": round(copy_gbps, 1), "frac_of_copy": round(step_gbps / copy_gbps, 4)},
        "timing": timing,
        "graph_warmup_replays": None if args.no_graph else max(args.warmup, GRAPH_WARMUP),
        "replay_us": replay_us,
        "per_kernel_us": per_kernel_us,
        "eager_ms_per_step": round(eager_ms, 5),
        "n_acc": step.n_acc.cpu().tolist()[:8],
        "roofline": roofline,
        "decode_loop": loop_rep,
        "full_depth": full_rep,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one step ...")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.mode, tau, eps, delta)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
