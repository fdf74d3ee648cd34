"""Benchmark of the hybrid Top-k + Top-p block-sparse attention path on one MI355X.

One step = the whole path on one batch of synthetic input: mask prediction
(pool Q and K, float64 block scores, hybrid selection, index list) and the
re-packing of V (on a second stream, after the pooling and beside the scores
and the selection), then the block-sparse attention forward over the kept key
blocks. Inputs are resident in HBM before the timed region starts. The step
time is the average over K steps replayed from a HIP graph of one step (every
launch and stream join of the step, nothing skipped; --no-graph times them
eagerly); the mask, pack and attention-kernel times come from an eager pass of
the same K steps with HIP events around each part.

Default workload: the Wan2.1-1.3B-shaped grid (B=1, H=12, N=32760 =
21x30x52, d=128, blocks 128x64, k=5%, p=0.9). `value` is dense-equivalent
throughput: 4*B*H*N^2*d floating-point operations per step divided by the
step time (TFLOP/s). Next to it the line reports the attention kernel against
the bf16 MFMA roofline at the kept-block count, the same path at the Top-k
operating points of 90% and 95% block sparsity (p = 0, k = 10% / 5%), the
backward, low-bit, sparse-linear, SLA2/SALAD and SVG2 variants on the same
inputs, the forward at two more configurations (95% sparsity on mixed-range
heads, and a Wan2.1-14B 720p grid: H=40, N=75600), and the CPU oracle timed on
a bounded sample of the default workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attn ms + dense-equiv TFLOPS (% bf16 MFMA peak) at 90/95% sparsity"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_softmax_amd", "csrc", "attn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_fwd_wan1.3b_traffic.txt")


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None if the kernel source changed since."""
    import hashlib
    try:
        kv = dict(line.split("=", 1) for line in open(TRAFFIC_FILE)
                  if "=" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        src = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
        if kv.get("kernel_source_sha256") != src:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def kept_flops(cnt: np.ndarray, idx: np.ndarray, N: int, d: int, block_q: int,
               block_k: int) -> float:
    """Algorithmic FLOPs of the attention over the kept tiles: for every kept
    (query block i, key block j), 4 * d * |I_i| * |J_j| with true token counts."""
    B, H, n_q = cnt.shape
    qrows = np.minimum(block_q, N - np.arange(n_q) * block_q).astype(np.float64)
    n_k = idx.shape[-1]
    krows = np.minimum(block_k, N - np.arange(n_k) * block_k).astype(np.float64)
    total = 0.0
    flat_c = cnt.reshape(-1, n_q)
    flat_i = idx.reshape(-1, n_q, n_k)
    for bh in range(flat_c.shape[0]):
        for i in range(n_q):
            c = flat_c[bh, i]
            total += qrows[i] * krows[flat_i[bh, i, :c]].sum()
    return 4.0 * d * total


def cpu_baseline(wl, Q, K, V, blocks: int):
    """The oracle, as it stands, on a bounded sample: heads 0, 1, ... in order,
    each with its whole mask and the masked attention of its query blocks, until
    `blocks` query blocks have been attended."""
    from oracle import sparge_oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t_mask = t_attn = 0.0
    rows = heads = done = 0
    for h in range(wl.H):
        if done >= blocks:
            break
        q, k, v = (O.bf16_to_f64(X[0, h]) for X in (Q, K, V))
        t0 = time.perf_counter()
        sel, _ = O.predict_mask_head(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass,
                                     wl.scale)
        t_mask += time.perf_counter() - t0
        nb = min(blocks - done, wl.n_q)
        t0 = time.perf_counter()
        O.masked_attention_head(q, k, v, sel.kept, wl.block_q, wl.block_k, wl.scale,
                                q_blocks=range(nb))
        t_attn += time.perf_counter() - t0
        rows += min(nb * wl.block_q, wl.N)
        done += nb
        heads += 1
    t = t_mask + t_attn
    dense = 4.0 * rows * wl.N * wl.d
    return {"value": dense / t / 1e12, "unit": "TFLOPS (dense-equivalent)", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{wl.name} heads 0-{heads - 1}: mask of every query block of each head "
                      f"({t_mask:.2f} s) + attention of {done} query blocks ({t_attn:.2f} s), "
                      f"float64 NumPy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan1.3b")
    ap.add_argument("--cpu-blocks", type=int, default=768,
                    help="query blocks of the oracle's CPU sample (heads 0, 1, ... in order)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the forward at the 95%% and Wan 14B 720p configurations")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time the plain step eagerly instead of replaying a HIP graph of it")
    ap.add_argument("--no-overlap", action="store_true",
                    help="pack V on the main stream between the mask's halves instead of beside "
                         "the second")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first, as a "
                         "known-size reference for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_attention_softmax_amd import binding as S
    from block_sparse_attention_softmax_amd.workloads import (WORKLOADS, generate, mix_alpha,
                                                              router_weights)

    wl = WORKLOADS[args.workload]
    Q, K, V = generate(wl)
    dev = torch.device("cuda:0")
    g = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
    q, k, v = g(Q), g(K), g(V)
    B, H, N, d = q.shape
    n_q, n_k = wl.n_q, wl.n_k
    bits = torch.empty((B, H, n_q, -(-n_k // 32)), dtype=torch.int32, device=dev)
    idx = torch.empty((B, H, n_q, n_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, n_q), dtype=torch.int32, device=dev)
    ws = torch.empty(S.mask_workspace_bytes(B, H, N, d, wl.block_q, wl.block_k),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    aws = torch.empty(S.attn_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    lws = torch.empty(S.linear_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    alpha = torch.full((H,), 0.1, dtype=torch.float32, device=dev)
    # SLA2 / SALAD variants: per-channel mix ratios, router weights, dropped branches
    alpha_mix = torch.from_numpy(mix_alpha(H, d, 5)).to(dev)
    alpha_half = torch.tensor([0.1 if h % 2 else 0.0 for h in range(H)], dtype=torch.float32,
                              device=dev)
    alpha_none = torch.zeros(H, dtype=torch.float32, device=dev)
    w_q, w_k = (torch.from_numpy(w).to(dev) for w in router_weights(H, d, 77))
    rws = torch.empty(S.mask_routed_workspace_bytes(B, H, N, d, wl.block_q, wl.block_k),
                      dtype=torch.uint8, device=dev)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority

    pooled = torch.cuda.Event()

    def step(k_frac, p_mass, ev=None, linear=None, alpha_t=None, routed=False):
        """mask pooling -> (V pack on the side stream || block scores and selection)
        -> attention, all but the pack on the main stream.

        Pooling and the V pack both stream a whole tensor from HBM, the scores
        and the selection do not, so the pack waits for the pooling and runs
        beside the rest of the mask. The pack's wait on the pooling also orders
        it after the previous step's attention, which reads the packed V. (The
        routed mask, kept in one call, runs beside the whole pack.)"""
        cur = torch.cuda.current_stream()  # the main stream, or the capture stream
        pack_stream = cur if args.no_overlap else side

        def pack():
            with torch.cuda.stream(pack_stream):
                if ev is not None:
                    ev[4].record()
                S.sparge_attn_pack(v, workspace=aws)
                if ev is not None:
                    ev[5].record()

        if routed:
            side.wait_stream(cur)
            pack()
            if ev is not None:
                ev[0].record()
            S.sparge_mask_predict_routed(q, k, w_q, w_k, wl.block_q, wl.block_k, k_frac, p_mass,
                                         wl.scale, workspace=rws, out=(bits, idx, cnt))
        else:
            if ev is not None:
                ev[0].record()
            S.sparge_mask_pool(q, k, wl.block_q, wl.block_k, workspace=ws)
            if not linear:
                pooled.record(cur)
                side.wait_event(pooled)
                pack()
            S.sparge_mask_select(q, ws, wl.block_q, wl.block_k, k_frac, p_mass, wl.scale,
                                 out=(bits, idx, cnt))
        if ev is not None:
            ev[1].record()
        if linear:
            fn = S.sla2_mix_attn_fwd if linear == "mix" else S.sparse_linear_attn_fwd
            fn(q, k, v, idx, cnt, alpha_t, wl.block_q, wl.block_k, wl.scale, workspace=lws,
               out=o)
            if ev is not None:
                ev[2].record()
        else:
            cur.wait_stream(side)
            if ev is not None:
                ev[2].record()
            S.sparge_attn_fwd_packed(q, k, idx, cnt, aws, wl.block_q, wl.block_k, wl.scale,
                                     out=o)
        if ev is not None:
            ev[3].record()

    def capture(fn):
        """A HIP graph of fn's launches (both streams), captured after one run on
        the capture stream."""
        graph, cs = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        cs.wait_stream(main)
        with torch.cuda.stream(cs):
            fn()
        main.wait_stream(cs)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cs):
            fn()
        return graph

    def timed(k_frac, p_mass, steps, warmup, linear=None, alpha_t=None, routed=False):
        kw = dict(linear=linear, alpha_t=alpha_t, routed=routed)
        for _ in range(warmup):
            step(k_frac, p_mass, **kw)
        torch.cuda.synchronize()
        # the breakdown: the steps once with events around their parts
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        for i in range(steps):
            step(k_frac, p_mass, evs[i], **kw)
        torch.cuda.synchronize()
        # the step time: the same steps without events; the plain path replayed
        # from a HIP graph of one step (its launches and stream joins)
        run = lambda: step(k_frac, p_mass, **kw)
        graph = None
        if args.graph and not linear and not routed:
            graph = capture(run)
            run = graph.replay
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        del graph
        mask_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        pack_ms = (float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) if linear else
                   float(np.mean([e[4].elapsed_time(e[5]) for e in evs])))
        attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
        c_np, i_np = cnt.cpu().numpy(), idx.cpu().numpy()
        kf = kept_flops(c_np, i_np, N, d, wl.block_q, wl.block_k)
        kept_frac = float(c_np.sum()) / (B * H * n_q * n_k)
        return wall, mask_ms, pack_ms, attn_ms, kf, kept_frac

    dense = 4.0 * B * H * float(N) * N * d
    wall, mask_ms, pack_ms, kern_ms, kf, kept_frac = timed(wl.k_frac, wl.p_mass, args.steps,
                                                            args.warmup)
    achieved = kf / (kern_ms * 1e-3) / 1e12

    points = {}
    for kfrac in (0.10, 0.05):
        w2, m2, p2, k2, kf2, frac2 = timed(kfrac, 0.0, max(5, args.steps // 2), 2)
        points[f"p0_k{int(kfrac * 100)}"] = {
            "k": kfrac, "p": 0.0, "block_sparsity": round(1 - frac2, 4),
            "ms_per_step": round(w2 * 1e3, 4), "mask_ms": round(m2, 4),
            "pack_ms": round(p2, 4), "attn_kernel_ms": round(k2, 4),
            "dense_equiv_tflops": round(dense / w2 / 1e12, 2),
            "attn_dense_equiv_tflops": round(dense / (k2 * 1e-3) / 1e12, 2),
            "attn_kept_tflops": round(kf2 / (k2 * 1e-3) / 1e12, 2),
            "attn_frac_bf16_peak": round(kf2 / (k2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}

    # the sparse-linear workload: same inputs and mask, plus alpha = 0.1 elu+1 linear branch
    n_lin = max(5, args.steps // 2)
    w3, m3, l3, _, kf3, frac3 = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="add",
                                      alpha_t=alpha)
    linear = {"workload": "wan1.3b_linear (alpha = 0.1, phi = elu + 1)",
              "ms_per_step": round(w3 * 1e3, 4), "mask_ms": round(m3, 4),
              "sparse_linear_ms": round(l3, 4),
              "dense_equiv_tflops": round(dense / w3 / 1e12, 2)}

    # SLA2: router mask (projected pooled Q, K; hard Top-k) and the per-channel mix;
    # SALAD: the added branch dropped on half of the heads, then on all of them
    w4, m4, _, _, _, frac4 = timed(0.10, 0.0, n_lin, 2, routed=True)
    w5, m5, l5, _, _, _ = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="mix",
                                alpha_t=alpha_mix)
    w6, _, l6, _, _, _ = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="add",
                               alpha_t=alpha_half)
    w7, _, l7, _, _, _ = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="add",
                               alpha_t=alpha_none)
    sla2 = {"routed_mask": {"k": 0.10, "p": 0.0, "weights": "N(0, 1/d) per head, float32",
                            "mask_ms": round(m4, 4), "ms_per_step": round(w4 * 1e3, 4),
                            "block_sparsity": round(1 - frac4, 4)},
            "mix": {"alpha": "uniform [0, 1) per head and channel",
                    "ms_per_step": round(w5 * 1e3, 4), "mix_attn_ms": round(l5, 4)},
            "drop_half": {"alpha": "0.1 on odd heads, 0 (dropped) on even heads",
                          "ms_per_step": round(w6 * 1e3, 4), "sparse_linear_ms": round(l6, 4)},
            "drop_all": {"alpha": "0 on every head (every branch dropped)",
                         "ms_per_step": round(w7 * 1e3, 4), "sparse_linear_ms": round(l7, 4)}}

    # backward of the sparse attention (dQ, dK, dV for a random dO), on the headline
    # mask and at the 95% point; the forward with log-sum-exp runs once, untimed
    d_o = torch.randn(q.shape, dtype=torch.float32, device=dev,
                      generator=torch.Generator(device=dev).manual_seed(3)).to(torch.bfloat16)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = [torch.empty_like(q) for _ in range(3)]
    bws = torch.empty(S.attn_bwd_workspace_bytes(B, H, N, d, wl.block_q, wl.block_k),
                      dtype=torch.uint8, device=dev)
    backward = {}
    for name, kfrac, pm, n_b in (("headline", wl.k_frac, wl.p_mass, max(3, args.steps // 5)),
                                 ("p0_k5", 0.05, 0.0, max(5, args.steps // 2))):
        S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, kfrac, pm, wl.scale, workspace=ws,
                              out=(bits, idx, cnt))
        S.sparge_attn_fwd_lse(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale, out=(o, lse),
                              workspace=aws)

        def bwd():
            S.sparge_attn_bwd(q, k, v, o, d_o, lse, idx, cnt, wl.block_q, wl.block_k, wl.scale,
                              out=grads, workspace=bws)
        bwd()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_b):
            bwd()
        e1.record()
        torch.cuda.synchronize()
        b_ms = e0.elapsed_time(e1) / n_b
        c_np, i_np = cnt.cpu().numpy(), idx.cpu().numpy()
        kfb = 2.5 * kept_flops(c_np, i_np, N, d, wl.block_q, wl.block_k)  # 5 products
        backward[name] = {"k": kfrac, "p": pm,
                          "block_sparsity": round(1 - float(c_np.sum()) / (B * H * n_q * n_k), 4),
                          "bwd_ms": round(b_ms, 4), "algorithmic_tflops": round(kfb / b_ms / 1e9, 2),
                          "frac_bf16_peak": round(kfb / b_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}

    # backward of the sparse-linear output (alpha = 0.1) on the headline mask
    S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass, wl.scale,
                          workspace=ws, out=(bits, idx, cnt))
    S.sparse_linear_attn_fwd(q, k, v, idx, cnt, alpha, wl.block_q, wl.block_k, wl.scale,
                             workspace=lws, out=o, lse=lse)
    lbws = torch.empty(S.linear_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def lbwd():
        S.sparse_linear_attn_bwd(q, k, v, o, d_o, lse, idx, cnt, alpha, wl.block_q, wl.block_k,
                                 wl.scale, out=grads, workspace=lbws)
    lbwd()
    torch.cuda.synchronize()
    n_b = max(3, args.steps // 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_b):
        lbwd()
    e1.record()
    torch.cuda.synchronize()
    backward["sparse_linear_headline"] = {
        "k": wl.k_frac, "p": wl.p_mass, "alpha": 0.1,
        "bwd_ms": round(e0.elapsed_time(e1) / n_b, 4),
        "vs_sparse_bwd": round(e0.elapsed_time(e1) / n_b / backward["headline"]["bwd_ms"], 3)}
    del lbws

    # the low-bit sparse branch (INT8 Q/K, e4m3 P/V) on the same masks: whole call
    # (quantisation of Q, K and V included) against the bf16 attention call
    lowbit = {}
    lws8 = torch.empty(S.lowbit_workspace_bytes(B, H, N, d, wl.block_q, wl.block_k),
                       dtype=torch.uint8, device=dev)
    for name, kfrac, pm in (("headline", wl.k_frac, wl.p_mass), ("p0_k10", 0.10, 0.0),
                            ("p0_k5", 0.05, 0.0)):
        S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, kfrac, pm, wl.scale, workspace=ws,
                              out=(bits, idx, cnt))
        c_np, i_np = cnt.cpu().numpy(), idx.cpu().numpy()
        kf_lb = kept_flops(c_np, i_np, N, d, wl.block_q, wl.block_k)
        res = {}
        for tag, fn in (("lowbit", lambda: S.sparge_attn_fwd_lowbit(
                             q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale, out=o,
                             workspace=lws8)),
                        ("bf16", lambda: S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q,
                                                           wl.block_k, wl.scale, out=o,
                                                           workspace=aws))):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n_l = max(5, args.steps // 2)
            e0.record()
            for _ in range(n_l):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[tag] = e0.elapsed_time(e1) / n_l
        lowbit[name] = {"k": kfrac, "p": pm, "lowbit_call_ms": round(res["lowbit"], 4),
                        "bf16_call_ms": round(res["bf16"], 4),
                        "lowbit_kept_tops": round(kf_lb / res["lowbit"] / 1e9, 1)}
    del lws8

    # SVG2's clustered attention (256 query / 512 key clusters, 3 k-means rounds, p = 0.9)
    sws = torch.empty(S.svg2_workspace_bytes(B, H, N, d, wl.block_q, 256, 512), dtype=torch.uint8,
                      device=dev)

    def svg2():
        S.svg2_attn_fwd(q, k, v, 256, 512, iters=3, p_mass=0.9, block_q=wl.block_q, scale=wl.scale,
                        out=o, workspace=sws)
    svg2()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        svg2()
    e1.record()
    torch.cuda.synchronize()
    svg2_line = {"clusters": [256, 512], "kmeans_rounds": 3, "p": 0.9,
                 "call_ms": round(e0.elapsed_time(e1) / 3, 3)}
    del sws

    # the forward at the two other configurations: 95% sparsity on mixed-range heads
    # (k = 3%, p = 0.8) and Wan 14B at 720p (H = 40, N = 75600); mask, V pack and the
    # attention kernel, each timed on its own over the same launches
    other = {}
    if not args.no_other_configs:
        for name in ("wan1.3b_s95", "wan14b_720p"):
            w2 = WORKLOADS[name]
            q2, k2, v2 = (g(a) for a in generate(w2))
            B2, H2, N2, d2 = q2.shape
            bits2 = torch.empty((B2, H2, w2.n_q, -(-w2.n_k // 32)), dtype=torch.int32,
                                device=dev)
            idx2 = torch.empty((B2, H2, w2.n_q, w2.n_k), dtype=torch.int32, device=dev)
            cnt2 = torch.empty((B2, H2, w2.n_q), dtype=torch.int32, device=dev)
            ws2 = torch.empty(S.mask_workspace_bytes(B2, H2, N2, d2, w2.block_q, w2.block_k),
                              dtype=torch.uint8, device=dev)
            aws2 = torch.empty(S.attn_workspace_bytes(B2, H2, N2, d2), dtype=torch.uint8,
                               device=dev)
            o2 = torch.empty_like(q2)

            def fwd2(ev=None):
                if ev is not None:
                    ev[0].record()
                S.sparge_mask_predict(q2, k2, w2.block_q, w2.block_k, w2.k_frac, w2.p_mass,
                                      w2.scale, workspace=ws2, out=(bits2, idx2, cnt2))
                if ev is not None:
                    ev[1].record()
                S.sparge_attn_pack(v2, workspace=aws2)
                if ev is not None:
                    ev[2].record()
                S.sparge_attn_fwd_packed(q2, k2, idx2, cnt2, aws2, w2.block_q, w2.block_k,
                                         w2.scale, out=o2)
                if ev is not None:
                    ev[3].record()
            fwd2()
            torch.cuda.synchronize()
            n_o = max(3, args.steps // 4)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_o)]
            for i in range(n_o):
                fwd2(evs[i])
            torch.cuda.synchronize()
            ms = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(3)]
            c_np, i_np = cnt2.cpu().numpy(), idx2.cpu().numpy()
            kf2 = kept_flops(c_np, i_np, N2, d2, w2.block_q, w2.block_k)
            dense2 = 4.0 * B2 * H2 * float(N2) * N2 * d2
            total = sum(ms)
            other[name] = {
                "shape": f"B={B2} H={H2} N={N2} d={d2} blocks {w2.block_q}x{w2.block_k}",
                "k": w2.k_frac, "p": w2.p_mass,
                "block_sparsity": round(1 - float(c_np.sum()) / c_np.size / w2.n_k, 4),
                "mask_ms": round(ms[0], 4), "pack_ms": round(ms[1], 4),
                "attn_kernel_ms": round(ms[2], 4), "sequential_ms": round(total, 4),
                "dense_equiv_tflops": round(dense2 / total / 1e9, 2),
                "attn_kept_tflops": round(kf2 / ms[2] / 1e9, 2),
                "attn_frac_bf16_peak": round(kf2 / ms[2] / 1e9 / PEAK_BF16_TFLOPS, 4)}
            del q2, k2, v2, bits2, idx2, cnt2, ws2, aws2, o2
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, Q, K, V, args.cpu_blocks)

    line = {
        "metric": METRIC,
        "value": round(dense / wall / 1e12, 3),
        "unit": "TFLOPS (dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={B} H={H} N={N} (grid {'x'.join(map(str, wl.grid))})"
                               f" d={d} blocks {wl.block_q}x{wl.block_k} k={wl.k_frac} "
                               f"p={wl.p_mass}",
                   "global_batch": B, "seq_len": N, "parallelism": "single GPU",
                   "block_sparsity": round(1 - kept_frac, 4)},
        "mask_ms": round(mask_ms, 4), "pack_ms": round(pack_ms, 4),
        "attn_kernel_ms": round(kern_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "sparse_attn_fwd_kernel<128,128,false>",
                     "flops_per_launch": kf},
        "operating_points": points,
        "sparse_linear": linear,
        "sla2_salad": sla2,
        "backward": backward,
        "lowbit": lowbit,
        "svg2": svg2_line,
        "other_configs": other,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
