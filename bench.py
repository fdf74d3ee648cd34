"""Benchmark of the hybrid Top-k + Top-p block-sparse attention path on one MI355X.

One step = the whole path on one batch of synthetic input: mask prediction
(pool Q and K, float64 block scores, hybrid selection, index list) and the
re-packing of V (on a second stream, after the pooling and beside the scores
and the selection), then the block-sparse attention forward over the kept key
blocks. Inputs are resident in HBM before the timed region starts. The step
time is the average over K steps replayed from a HIP graph of one step (every
launch and stream join of the step, nothing skipped; --no-graph times them
eagerly); the mask, pack and attention-kernel times come from an eager pass of
the same K steps with HIP events around each part; the median, 10th and 90th
percentile of the step come from the same steps timed one by one, and a "cold"
pass times each step again after writing 512 MiB (more than the Infinity
Cache holds) so that it starts from HBM.

Default workload: the Wan2.1-1.3B-shaped grid (B=1, H=12, N=32760 =
21x30x52, d=128, blocks 128x64, k=5%, p=0.9). `value` is dense-equivalent
throughput: 4*B*H*N^2*d floating-point operations per step divided by the
step time (TFLOP/s). Next to it the line reports the attention kernel against
the bf16 MFMA roofline at the kept-block count, the same path at the Top-k
operating points of 90% and 95% block sparsity (p = 0, k = 10% / 5%), the
backward, low-bit, sparse-linear, SLA2/SALAD and SVG2 variants on the same
inputs, the forward at two more configurations (95% sparsity on mixed-range
heads, and a Wan2.1-14B 720p grid: H=40, N=75600, and the tiny case), the
measured MFMA and HBM ceilings, and the CPU oracle timed on a bounded sample
of the default workload, followed (untimed) by the oracle's check of the
benchmarked masks and of sampled output rows for every configuration.

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


_T0 = time.perf_counter()


def progress(phase: str):
    """One line on stderr as each part of the run ends (the JSON line stays alone on stdout)."""
    print(f"bench: {phase} done at {time.perf_counter() - _T0:.0f} s", file=sys.stderr, flush=True)


def dist(ms) -> dict:
    """Median, 10th and 90th percentile of a list of times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def host_info() -> dict:
    """The host the oracle runs on: core counts, CPU model, BLAS threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model,
            "blas_threads": blas}


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

    host = host_info()
    cores = host["blas_threads"] or host["affinity_cpus"] or host["nproc"] or 1
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
                      f"float64 NumPy",
            "host": host, "mask_s": round(t_mask, 3), "attn_s": round(t_attn, 3)}


def measure_ceilings(torch, dev) -> dict:
    """The dense bf16 MFMA rate the probe kernel sustains (TFLOP/s; the better of
    4 and 8 independent chains per wave) and the HBM bandwidth of a 1 GiB
    device-to-device copy (GB/s, read + write bytes)."""
    import ctypes
    out = {"mfma_bf16_tflops": None, "hbm_copy_gbs": None}
    probe = os.path.join(ROOT, "block_sparse_attention_softmax_amd", "libsparge_probe.so")
    L = ctypes.CDLL(probe)
    L.sparge_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    L.sparge_probe_mfma_bf16.restype = ctypes.c_int
    L.sparge_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.sparge_probe_mfma_flops.restype = ctypes.c_double
    blocks, iters = 256 * 2 * 8, 8192  # 8 waves per CU, 8 rounds of the chip
    buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = []
    for chains in (4, 8):
        rates = []
        for rep in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = L.sparge_probe_mfma_bf16(ctypes.c_void_p(buf.data_ptr()), blocks, iters, chains,
                                          st)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"MFMA probe launch failed: HIP error {rc}")
            if rep:  # the first launch warms the clock and loads the code
                rates.append(L.sparge_probe_mfma_flops(blocks, iters, chains) /
                             (e0.elapsed_time(e1) * 1e9))
        best.append(float(np.median(rates)))
    out["mfma_bf16_tflops"] = round(max(best), 1)
    out["mfma_bf16_tflops_4_8_chains"] = [round(x, 1) for x in best]
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    gbs = []
    for rep in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            gbs.append(2.0 * src.numel() / (e0.elapsed_time(e1) * 1e6))
    out["hbm_copy_gbs"] = round(float(np.median(gbs)), 1)
    del src, dst, buf
    torch.cuda.empty_cache()
    return out


def oracle_check(samples, inputs) -> dict:
    """Untimed parity check of the benchmarked GPU results against the oracle,
    per configuration: the oracle's mask over every row (its near-tie rows, and
    rows where the GPU's mask differs) and the oracle's attention on the seeded
    sample of query blocks the GPU output was kept for (max / mean abs error)."""
    from oracle import sparge_oracle as O

    out = {}
    masks = {}
    for smp in samples:
        wl = smp["wl"]
        Q, K, V = inputs[smp["inputs"]]
        key = (smp["inputs"], smp["k"], smp["p"])
        if key not in masks:
            masks[key] = O.predict_mask(Q, K, wl.block_q, wl.block_k, smp["k"], smp["p"],
                                        wl.scale)
        m = masks[key]
        j = np.arange(wl.n_k)
        gpu_kept = ((smp["bits"][..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)
        rows_differ = int((gpu_kept != m.kept).any(-1).sum())
        errs = []
        for h, blocks, got in smp["rows"]:
            q, k, v = (O.bf16_to_f64(X[0, h]) for X in (Q, K, V))
            if smp["alpha"] is None:
                ref = O.masked_attention_head(q, k, v, m.kept[0, h], wl.block_q, wl.block_k,
                                              wl.scale, q_blocks=blocks)
            else:
                ref = O.sparse_linear_attention_head(q, k, v, m.kept[0, h], wl.block_q,
                                                     wl.block_k, wl.scale, smp["alpha"],
                                                     q_blocks=blocks)
            valid = ~np.isnan(ref[:, 0])
            errs.append(np.abs(O.bf16_to_f64(got) - ref[valid]))
        e = np.concatenate([x.ravel() for x in errs])
        out[smp["name"]] = {
            "mask_rows": int(m.kept[..., 0].size), "near_tie_rows": int((m.margin < 1e-5).sum()),
            "rows_differing_from_oracle": rows_differ,
            "output_sample": f"{sum(len(b) for _, b, _ in smp['rows'])} query blocks of heads "
                             f"{[h for h, _, _ in smp['rows']]}",
            "max_abs_err": float(e.max()), "mean_abs_err": float(e.mean())}
    return out


def svg2_measure(S, q, k, v, o, ws, wl, cq, ck, iters, p_mass, reps=3):
    """SVG2 call, clustering and attention times and the token-pair counts."""
    import torch
    B, H, N, d = q.shape

    def med(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))
    call = med(lambda: S.svg2_attn_fwd(q, k, v, cq, ck, iters=iters, p_mass=p_mass,
                                       block_q=wl.block_q, scale=wl.scale, out=o, workspace=ws))
    clus = med(lambda: S.svg2_attn_cluster(q, k, v, cq, ck, iters=iters, p_mass=p_mass,
                                           block_q=wl.block_q, scale=wl.scale, workspace=ws))
    att = med(lambda: S.svg2_attn_apply(q, cq, ck, ws, wl.block_q, wl.scale, out=o))
    counts = S.svg2_attn_pair_counts(q, cq, ck, ws, wl.block_q).cpu().numpy()
    useful, computed = float(counts[..., 0].sum()), float(counts[..., 1].sum())
    tf_useful = 4.0 * d * useful / (att * 1e-3) / 1e12
    return {"clusters": [cq, ck], "kmeans_rounds": iters, "p": p_mass,
            "call_ms": round(call, 3), "cluster_ms": round(clus, 3), "attn_ms": round(att, 3),
            "token_density": round(useful / (B * H * float(N) * N), 4),
            "useful_pairs": useful, "computed_pairs": computed,
            "padding_share": round(1.0 - useful / computed, 4),
            "attn_useful_tflops": round(tf_useful, 1),
            "attn_useful_frac_bf16_peak": round(tf_useful / PEAK_BF16_TFLOPS, 4),
            "attn_computed_tflops": round(4.0 * d * computed / (att * 1e-3) / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
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
    ap.add_argument("--svg2", action="store_true",
                    help="time only the SVG2 call and its parts on the workload (for profiling) "
                         "and print its line")
    ap.add_argument("--point", default=None, metavar="K,P",
                    help="time only the forward step at Top-k fraction K and Top-p mass P on the "
                         "workload (for profiling one operating point) and print its line")
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

    def gpu_sample(name, w, k_frac, p_mass, bits_t, o_t, alpha=None, inputs=None):
        """Copies, outside every timed region, of a benchmarked GPU mask and of
        its output rows on a seeded sample of query blocks (first, last and four
        more, on two heads: for the mixed-range configuration one near-uniform
        and one sink head), for the oracle check."""
        rng = np.random.default_rng(len(name) + int(k_frac * 1000))
        if w.name == "wan1.3b_s95":
            heads = [int(rng.integers(0, w.H // 2)), int(rng.integers(w.H // 2, w.H))]
        else:
            heads = sorted(int(h) for h in rng.choice(w.H, size=min(2, w.H), replace=False))
        rows = []
        for h in heads:
            blocks = sorted({0, w.n_q - 1, *(int(b) for b in rng.choice(w.n_q, min(4, w.n_q),
                                                                          replace=False))})
            sel = np.concatenate([np.arange(b * w.block_q, min((b + 1) * w.block_q, w.N))
                                  for b in blocks])
            got = o_t[0, h][torch.from_numpy(sel).to(o_t.device)]
            rows.append((h, blocks, got.cpu().view(torch.uint16).numpy()))
        return {"name": name, "wl": w, "inputs": inputs or w.name, "k": k_frac, "p": p_mass,
                "alpha": alpha, "bits": bits_t.cpu().numpy().view(np.uint32), "rows": rows}

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

    # writing this between repetitions evicts the 256 MiB Infinity Cache (MALL)
    # and every L2, so the next step starts from HBM ("cold")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timed(k_frac, p_mass, steps, warmup, linear=None, alpha_t=None, routed=False,
              cold=False):
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
        # the distribution: each step of the same kind between two events
        se = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in se:
            e[0].record()
            run()
            e[1].record()
        torch.cuda.synchronize()
        del graph
        mask = [e[0].elapsed_time(e[1]) for e in evs]
        pack = ([e[1].elapsed_time(e[2]) for e in evs] if linear else
                [e[4].elapsed_time(e[5]) for e in evs])
        attn = [e[2].elapsed_time(e[3]) for e in evs]
        r = {"wall": wall, "mask_ms": float(np.mean(mask)), "pack_ms": float(np.mean(pack)),
             "attn_ms": float(np.mean(attn)), "step_dist": dist([a.elapsed_time(b) for a, b in se]),
             "attn_dist": dist(attn)}
        if cold:
            # each step after the cache flush: eager, events around its parts
            ce = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
            for i in range(steps):
                flush.fill_(i & 0xFF)
                step(k_frac, p_mass, ce[i], **kw)
            torch.cuda.synchronize()
            r["cold"] = {"step_ms": dist([e[0].elapsed_time(e[3]) for e in ce]),
                         "mask_ms": dist([e[0].elapsed_time(e[1]) for e in ce]),
                         "attn_kernel_ms": dist([e[2].elapsed_time(e[3]) for e in ce])}
        c_np, i_np = cnt.cpu().numpy(), idx.cpu().numpy()
        r["kf"] = kept_flops(c_np, i_np, N, d, wl.block_q, wl.block_k)
        r["kept_frac"] = float(c_np.sum()) / (B * H * n_q * n_k)
        return r

    if args.svg2:
        sws = torch.empty(S.svg2_workspace_bytes(B, H, N, d, wl.block_q, 256, 512),
                          dtype=torch.uint8, device=dev)
        print(json.dumps({"workload": wl.name, **svg2_measure(S, q, k, v, o, sws, wl, 256, 512, 3,
                                                                0.9, reps=max(3, args.steps // 10))}),
              flush=True)
        return
    if args.point:
        kp, pp = (float(x) for x in args.point.split(","))
        r = timed(kp, pp, args.steps, args.warmup)
        tf = r["kf"] / (r["attn_ms"] * 1e-3) / 1e12
        print(json.dumps({"workload": wl.name, "k": kp, "p": pp, "steps": args.steps,
                          "block_sparsity": round(1 - r["kept_frac"], 4),
                          "ms_per_step": round(r["wall"] * 1e3, 4),
                          "attn_kernel_ms": round(r["attn_ms"], 4),
                          "attn_kernel_ms_dist": r["attn_dist"], "flops_per_launch": r["kf"],
                          "attn_kept_tflops": round(tf, 2),
                          "attn_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
        return

    progress("headline step")

    # measured ceilings beside the nameplate figures: dense bf16 MFMA (a probe
    # kernel of independent 32x32x16 chains) and HBM (a 1 GiB device copy)
    ceilings = measure_ceilings(torch, dev)

    dense = 4.0 * B * H * float(N) * N * d
    head = timed(wl.k_frac, wl.p_mass, args.steps, args.warmup, cold=True)
    wall, mask_ms, pack_ms, kern_ms = head["wall"], head["mask_ms"], head["pack_ms"], head["attn_ms"]
    kf, kept_frac = head["kf"], head["kept_frac"]
    achieved = kf / (kern_ms * 1e-3) / 1e12
    checks = [gpu_sample("wan1.3b", wl, wl.k_frac, wl.p_mass, bits, o)]

    points = {}
    for kfrac in (0.10, 0.05):
        r2 = timed(kfrac, 0.0, args.steps, 2, cold=True)
        w2, k2, kf2 = r2["wall"], r2["attn_ms"], r2["kf"]
        tf2 = kf2 / (k2 * 1e-3) / 1e12
        points[f"p0_k{int(kfrac * 100)}"] = {
            "k": kfrac, "p": 0.0, "block_sparsity": round(1 - r2["kept_frac"], 4),
            "ms_per_step": round(w2 * 1e3, 4), "mask_ms": round(r2["mask_ms"], 4),
            "pack_ms": round(r2["pack_ms"], 4), "attn_kernel_ms": round(k2, 4),
            "step_ms_dist": r2["step_dist"], "attn_kernel_ms_dist": r2["attn_dist"],
            "dense_equiv_tflops": round(dense / w2 / 1e12, 2),
            "attn_dense_equiv_tflops": round(dense / (k2 * 1e-3) / 1e12, 2),
            "attn_kept_tflops": round(tf2, 2),
            "attn_frac_bf16_peak": round(tf2 / PEAK_BF16_TFLOPS, 4),
            "attn_frac_measured_mfma": round(tf2 / ceilings["mfma_bf16_tflops"], 4),
            "flops_per_launch": kf2, "cold": r2["cold"]}
        checks.append(gpu_sample(f"wan1.3b p=0 k={kfrac}", wl, kfrac, 0.0, bits, o))

    progress("ceilings and operating points")

    # the sparse-linear workload: same inputs and mask, plus alpha = 0.1 elu+1 linear branch
    n_lin = max(5, args.steps // 4)
    r3 = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="add", alpha_t=alpha)
    w3 = r3["wall"]
    linear = {"workload": "wan1.3b_linear (alpha = 0.1, phi = elu + 1)",
              "ms_per_step": round(w3 * 1e3, 4), "mask_ms": round(r3["mask_ms"], 4),
              "sparse_linear_ms": round(r3["pack_ms"], 4), "step_ms_dist": r3["step_dist"],
              "dense_equiv_tflops": round(dense / w3 / 1e12, 2)}
    checks.append(gpu_sample("wan1.3b_linear", WORKLOADS["wan1.3b_linear"], wl.k_frac, wl.p_mass,
                             bits, o, alpha=0.1, inputs=wl.name))

    progress("sparse-linear")

    # SLA2: router mask (projected pooled Q, K; hard Top-k) and the per-channel mix;
    # SALAD: the added branch dropped on half of the heads, then on all of them
    r4 = timed(0.10, 0.0, n_lin, 2, routed=True)
    w4, m4, frac4 = r4["wall"], r4["mask_ms"], r4["kept_frac"]
    r5 = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="mix", alpha_t=alpha_mix)
    w5, l5 = r5["wall"], r5["pack_ms"]
    r6 = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="add", alpha_t=alpha_half)
    w6, l6 = r6["wall"], r6["pack_ms"]
    r7 = timed(wl.k_frac, wl.p_mass, n_lin, 2, linear="add", alpha_t=alpha_none)
    w7, l7 = r7["wall"], r7["pack_ms"]
    sla2 = {"routed_mask": {"k": 0.10, "p": 0.0, "weights": "N(0, 1/d) per head, float32",
                            "mask_ms": round(m4, 4), "ms_per_step": round(w4 * 1e3, 4),
                            "block_sparsity": round(1 - frac4, 4)},
            "mix": {"alpha": "uniform [0, 1) per head and channel",
                    "ms_per_step": round(w5 * 1e3, 4), "mix_attn_ms": round(l5, 4)},
            "drop_half": {"alpha": "0.1 on odd heads, 0 (dropped) on even heads",
                          "ms_per_step": round(w6 * 1e3, 4), "sparse_linear_ms": round(l6, 4)},
            "drop_all": {"alpha": "0 on every head (every branch dropped)",
                         "ms_per_step": round(w7 * 1e3, 4), "sparse_linear_ms": round(l7, 4)}}

    progress("SLA2 / SALAD")

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

    progress("sparse backward")

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

    progress("sparse-linear backward")

    # the low-bit sparse branch (INT8 Q/K, e4m3 P/V) on the same masks. Its Q and K
    # codes come from the mask's pooling pass (sparge_mask_pool_lowbit), which
    # streams those blocks anyway; the attention call is then the V pack and the
    # kernel, as the bf16 call is the bf16 V pack and its kernel. Also timed: both
    # kernels alone, the pooling with and without the codes, the whole step of
    # each kind (pooling, selection, pack, attention, eager, in that order) and
    # the one-call form that quantises Q and K itself.
    def med(fn, n):
        fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for e in evs:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    lowbit = {}
    lws8 = torch.empty(S.lowbit_workspace_bytes(B, H, N, d, wl.block_q, wl.block_k),
                       dtype=torch.uint8, device=dev)
    for name, kfrac, pm in (("headline", wl.k_frac, wl.p_mass), ("p0_k10", 0.10, 0.0),
                            ("p0_k5", 0.05, 0.0)):
        S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, kfrac, pm, wl.scale, workspace=ws,
                              out=(bits, idx, cnt))
        c_np, i_np = cnt.cpu().numpy(), idx.cpu().numpy()
        kf_lb = kept_flops(c_np, i_np, N, d, wl.block_q, wl.block_k)
        n_l = max(5, args.steps // 2) if name != "headline" else max(3, args.steps // 5)
        S.sparge_mask_pool_lowbit(q, k, wl.block_q, wl.block_k, workspace=ws,
                                  lowbit_workspace=lws8)
        S.sparge_attn_lowbit_pack(v, lws8, wl.block_q)

        def lb_call():
            S.sparge_attn_lowbit_pack(v, lws8, wl.block_q)
            S.sparge_attn_fwd_lowbit_packed(q, idx, cnt, lws8, wl.block_q, wl.block_k, wl.scale,
                                            out=o)

        def lb_step():
            S.sparge_mask_pool_lowbit(q, k, wl.block_q, wl.block_k, workspace=ws,
                                      lowbit_workspace=lws8)
            S.sparge_mask_select(q, ws, wl.block_q, wl.block_k, kfrac, pm, wl.scale,
                                 out=(bits, idx, cnt))
            lb_call()

        def bf_step():
            S.sparge_mask_pool(q, k, wl.block_q, wl.block_k, workspace=ws)
            S.sparge_mask_select(q, ws, wl.block_q, wl.block_k, kfrac, pm, wl.scale,
                                 out=(bits, idx, cnt))
            S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale, out=o,
                              workspace=aws)
        t = {
            "lowbit_call_ms": med(lb_call, n_l),
            "bf16_call_ms": med(lambda: S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q,
                                                          wl.block_k, wl.scale, out=o,
                                                          workspace=aws), n_l),
            "lowbit_kernel_ms": med(lambda: S.sparge_attn_fwd_lowbit_packed(
                q, idx, cnt, lws8, wl.block_q, wl.block_k, wl.scale, out=o), n_l),
            "bf16_kernel_ms": med(lambda: S.sparge_attn_fwd_packed(
                q, k, idx, cnt, aws, wl.block_q, wl.block_k, wl.scale, out=o), n_l),
            "pool_lowbit_ms": med(lambda: S.sparge_mask_pool_lowbit(
                q, k, wl.block_q, wl.block_k, workspace=ws, lowbit_workspace=lws8), n_l),
            "pool_ms": med(lambda: S.sparge_mask_pool(q, k, wl.block_q, wl.block_k,
                                                      workspace=ws), n_l),
            "lowbit_step_ms": med(lb_step, n_l),
            "bf16_step_ms": med(bf_step, n_l),
            "one_call_lowbit_ms": med(lambda: S.sparge_attn_fwd_lowbit(
                q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale, out=o, workspace=lws8),
                n_l)}
        lowbit[name] = {"k": kfrac, "p": pm, **{key: round(x, 4) for key, x in t.items()},
                        "call_speedup": round(t["bf16_call_ms"] / t["lowbit_call_ms"], 3),
                        "step_speedup": round(t["bf16_step_ms"] / t["lowbit_step_ms"], 3),
                        "lowbit_kept_tops": round(kf_lb / t["lowbit_kernel_ms"] / 1e9, 1)}
    del lws8

    progress("low-bit")

    # SVG2's clustered attention (256 query / 512 key clusters, 3 k-means rounds, p = 0.9):
    # the whole call, and its two parts (clustering with the gathers; the attention
    # over the clusters, timed on its own with HIP events), with the token pairs
    # that take part and those the attention kernel evaluates (padding included)
    sws = torch.empty(S.svg2_workspace_bytes(B, H, N, d, wl.block_q, 256, 512), dtype=torch.uint8,
                      device=dev)
    svg2_line = svg2_measure(S, q, k, v, o, sws, wl, 256, 512, 3, 0.9)
    del sws

    progress("SVG2")

    # the forward at the other configurations: the tiny case, 95% sparsity on
    # mixed-range heads (k = 3%, p = 0.8) and Wan 14B at 720p (H = 40, N = 75600);
    # mask, V pack and the attention kernel, each timed on its own over the same
    # launches
    other = {}
    inputs = {wl.name: (Q, K, V)}
    if not args.no_other_configs:
        for name in ("tiny", "wan1.3b_s95", "wan14b_720p"):
            w2 = WORKLOADS[name]
            arrays = generate(w2)
            inputs[name] = arrays
            q2, k2, v2 = (g(a) for a in arrays)
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
            n_o = max(3, args.steps // 4) if name == "wan14b_720p" else args.steps
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_o)]
            for i in range(n_o):
                fwd2(evs[i])
            torch.cuda.synchronize()
            ms = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(3)]
            checks.append(gpu_sample(name, w2, w2.k_frac, w2.p_mass, bits2, o2))
            progress(f"forward at {name}")
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
                "attn_kernel_ms_dist": dist([e[2].elapsed_time(e[3]) for e in evs]),
                "dense_equiv_tflops": round(dense2 / total / 1e9, 2),
                "attn_kept_tflops": round(kf2 / ms[2] / 1e9, 2),
                "attn_frac_bf16_peak": round(kf2 / ms[2] / 1e9 / PEAK_BF16_TFLOPS, 4)}
            del q2, k2, v2, bits2, idx2, cnt2, ws2, aws2, o2
            torch.cuda.empty_cache()

    cpu = check = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, Q, K, V, args.cpu_blocks)
        progress("cpu baseline")
        t0 = time.perf_counter()
        check = oracle_check(checks, inputs)
        check["seconds"] = round(time.perf_counter() - t0, 1)

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
        "step_ms_dist": head["step_dist"], "attn_kernel_ms_dist": head["attn_dist"],
        "cold": head["cold"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "sparse_attn_fwd_kernel<128,128,false>",
                     "flops_per_launch": kf,
                     "measured_ceiling": ceilings["mfma_bf16_tflops"],
                     "frac_measured_ceiling": round(achieved / ceilings["mfma_bf16_tflops"], 4)},
        "ceilings": ceilings,
        "operating_points": points,
        "sparse_linear": linear,
        "sla2_salad": sla2,
        "backward": backward,
        "lowbit": lowbit,
        "svg2": svg2_line,
        "other_configs": other,
        "cpu_baseline": cpu,
        "oracle_check": check,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
