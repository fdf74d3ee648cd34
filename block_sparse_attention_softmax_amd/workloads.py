"""Seeded synthetic inputs shaped like the video-DiT attention workloads.

This module holds none of the method's arithmetic (no pooling, scoring,
selection or attention). It only draws random tensors and casts them to
bfloat16 bit patterns, so that the GPU path and the CPU oracle see exactly the
same bytes.

The workloads stand in for the Wan2.1 480p/720p latent grids that the
SpargeAttention2 page evaluates on (page "SpargeAttention2: Trainable Sparse
Attention via Hybrid Top-k+Top-p Masking and Distillation Fine-Tuning",
section 4, experimental results). The models, prompts and videos are not
available, so the recipe below stands in for them:

* tokens are a flattened T x Hg x W latent grid, time-major:
  u = (t * Hg + h) * W + w;
* "smooth" heads: one field F per head, N(0,1) per channel blurred over the
  grid with a Gaussian (sigma = 3 tokens, truncate 4, reflect boundary), then
  re-standardised per channel to zero mean and unit std; Q = F + 0.3 n_q,
  K = F + 0.3 n_k with independent N(0,1) noises, V ~ N(0,1);
* "sink" workloads add a scaled unit vector c to Q rows and to the first 64
  K rows, which makes one key block dominate the pooled scores;
* every head draws from its own PCG64 stream, spawned from the workload seed
  with numpy's SeedSequence (so heads can be drawn in parallel and any head
  can be regenerated alone); the sink vector c comes from one more stream;
* values are drawn in float64, rounded to float32, then to bfloat16 with
  round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    grid: tuple  # (T, Hg, W); N = T * Hg * W
    d: int
    block_q: int
    block_k: int
    k_frac: float
    p_mass: float
    seed: int
    kind: str  # "iid_sink" | "smooth" | "smooth_mixed"
    sink_gain: float = 0.0
    linear_alpha: float | None = None  # per-head alpha of the linear branch

    @property
    def N(self) -> int:
        return int(self.grid[0] * self.grid[1] * self.grid[2])

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32, as the C ABI receives it."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def n_q(self) -> int:
        return -(-self.N // self.block_q)

    @property
    def n_k(self) -> int:
        return -(-self.N // self.block_k)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, (4, 16, 16), 64, 64, 64, 0.10, 0.9, 0,
                     "iid_sink", sink_gain=4.0),
    "wan1.3b": Workload("wan1.3b", 1, 12, (21, 30, 52), 128, 128, 64, 0.05,
                        0.9, 1, "smooth"),
    "wan1.3b_s95": Workload("wan1.3b_s95", 1, 12, (21, 30, 52), 128, 128, 64,
                            0.03, 0.8, 2, "smooth_mixed", sink_gain=6.0),
    "wan14b_720p": Workload("wan14b_720p", 1, 40, (21, 45, 80), 128, 128, 64,
                            0.05, 0.9, 3, "smooth"),
    # same inputs as wan1.3b (seed 1), plus the linear branch on dropped blocks
    "wan1.3b_linear": Workload("wan1.3b_linear", 1, 12, (21, 30, 52), 128,
                               128, 64, 0.05, 0.9, 1, "smooth",
                               linear_alpha=0.1),
}
# The five workloads in the order the configuration table lists them.
WORKLOAD_ORDER = ["tiny", "wan1.3b", "wan1.3b_s95", "wan14b_720p",
                  "wan1.3b_linear"]


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _gaussian_field(rng: np.random.Generator, grid, d: int) -> np.ndarray:
    from scipy.ndimage import gaussian_filter

    T, Hg, W = grid
    raw = rng.standard_normal((T, Hg, W, d))
    f = gaussian_filter(raw, sigma=(3.0, 3.0, 3.0, 0.0), mode="reflect",
                        truncate=4.0)
    f = f.reshape(T * Hg * W, d)
    f -= f.mean(axis=0, keepdims=True)
    f /= f.std(axis=0, keepdims=True)
    return f


def _draw_head(wl: Workload, ss: np.random.SeedSequence):
    """One head's (Q, K, V) in float64, before any sink is added."""
    rng = np.random.Generator(np.random.PCG64(ss))
    N, d = wl.N, wl.d
    if wl.kind == "iid_sink":
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        return q, k, v
    f = _gaussian_field(rng, wl.grid, d)
    q = f + 0.3 * rng.standard_normal((N, d))
    k = f + 0.3 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    return q, k, v


def _sink_vector(wl: Workload, ss: np.random.SeedSequence) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(ss))
    g = rng.standard_normal(wl.d)
    return g / np.linalg.norm(g)


def generate_head(wl: Workload, b: int, h: int):
    """bf16 bit patterns (uint16 [N, d]) of Q, K, V for one (batch, head)."""
    children = np.random.SeedSequence(wl.seed).spawn(wl.B * wl.H + 1)
    q, k, v = _draw_head(wl, children[b * wl.H + h])
    if wl.kind in ("iid_sink", "smooth_mixed"):
        c = _sink_vector(wl, children[-1])
        if wl.kind == "iid_sink":
            q += wl.sink_gain * c
            k[0:64] += wl.sink_gain * c
        else:  # first half of the heads near-uniform, second half sinked
            if h < wl.H // 2:
                q *= 0.1
            else:
                q += wl.sink_gain * c
                k[0:64] += wl.sink_gain * c
    return f64_to_bf16_bits(q), f64_to_bf16_bits(k), f64_to_bf16_bits(v)


def generate(wl: Workload, threads: int | None = None):
    """Full (Q, K, V) as uint16 bf16 bit arrays of shape [B, H, N, d]."""
    shape = (wl.B, wl.H, wl.N, wl.d)
    Q = np.empty(shape, np.uint16)
    K = np.empty(shape, np.uint16)
    V = np.empty(shape, np.uint16)
    jobs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    if threads is None:
        threads = min(8, os.cpu_count() or 1)

    def one(job):
        b, h = job
        Q[b, h], K[b, h], V[b, h] = generate_head(wl, b, h)

    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, jobs))
    return Q, K, V


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def router_weights(H: int, d: int, seed: int) -> tuple:
    """Synthetic weights for the router's two projections (trained weights are
    not available): float32 [H, d, d] each, entries N(0, 1) / sqrt(d) from a
    PCG64 stream of `seed` (W_q drawn first, then W_k)."""
    rng = np.random.default_rng(seed)
    wq = (rng.standard_normal((H, d, d)) / np.sqrt(d)).astype(np.float32)
    wk = (rng.standard_normal((H, d, d)) / np.sqrt(d)).astype(np.float32)
    return wq, wk


def mix_alpha(H: int, d: int, seed: int) -> np.ndarray:
    """Synthetic learned ratios of the sparse / linear mix (trained values are
    not available): float32 [H, d], uniform in [0, 1) from a PCG64 stream of
    `seed`."""
    return np.random.default_rng(seed).random((H, d)).astype(np.float32)
