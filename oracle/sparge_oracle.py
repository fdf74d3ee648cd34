"""CPU oracle for hybrid Top-k + Top-p block-sparse attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library; the two meet only through the
seeded inputs of ``block_sparse_attention_softmax_amd.workloads``.

What it computes, step by step, in float64 with NumPy, written from the pages:

1. decode bfloat16 bit patterns exactly to float64;
2. mean-pool every block of query rows and of key rows (pooled queries and
   keys: "SLA2: Sparse-Linear Attention with Learnable Routing and QAT",
   sections 1 and 2B; block aggregates by mean pooling: "Sparse VideoGen2",
   section 1);
3. compressed block scores s = scale * Qbar Kbar^T and their row softmax
   (SLA2 page, section 2B, the compressed attention score; the same scale
   1/sqrt(d) as the attention itself);
4. order each row by score, highest first, ties to the lower block index;
5. Top-k keeps the first K_k entries of that order; Top-p keeps the shortest
   prefix whose cumulative probability reaches p ("SpargeAttention2: Trainable
   Sparse Attention via Hybrid Top-k+Top-p Masking and Distillation
   Fine-Tuning", section 1; "Sparse VideoGen2", section 2B);
6. the kept set is the union of the two (SpargeAttention2 page, section 2A);
   both are prefixes of one order, so the union is the longer prefix;
7. attention is plain softmax attention in which every key of a dropped block
   is masked out (the block-sparse kernel of SpargeAttention2 page, section 2C,
   only skips work that the mask removes, so its result is this);
8. optional linear branch over the dropped keys with phi = elu + 1, added to
   the sparse output with a per-head weight alpha (the SLA2 page, section 1,
   and the SALAD page's static scaling of the linear branch);
9. the SLA2 variants: the router's learnable linear projections of the pooled
   queries and keys before the compressed score (SLA2 page, section 2B; hard
   Top-k at inference, section 2D), and the faithful mix O = alpha (*) O_s +
   (1 - alpha) (*) O_l with a learned vector alpha in [0, 1] (section 2A);
10. post-tuning branch dropping (SALAD page): a head whose linear branch
   carries only small weights loses the branch, and its output is what the
   formula gives with the linear term removed;
11. the backward of step 7 (the sparse attention is fine-tuned, SpargeAttention2
   page, section 2B, so gradients pass through it): the log-sum-exp of every
   row's kept scores, and dQ, dK, dV of O = softmax(scale Q K^T, dropped keys
   masked) V for an upstream gradient dO, written out as the chain rule.

Readings of points the pages leave open (each also listed in the design
notes): mean pooling over the valid tokens of a partial last block; no
correction of the short last key block's score; K_k = min(n_k, max(1,
ceil(k * n_k - 1e-6))) computed from the float32 value of k; Top-p keeps the
block that crosses p (C_m >= p) and p >= 1 keeps every block; rows whose kept
list is empty produce zeros; the linear branch's phi is applied to the
unscaled Q and K and its output is zero when no block was dropped; alpha of
the mix is one value per output channel of a head; a branch counts as small
when every one of its weights (alpha[h] of the added form, 1 - alpha[h, c] of
the mix, each taken in float32) has magnitude <= a caller's threshold tau.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

NEAR_TIE_MARGIN = 1e-5


# ----------------------------------------------------------------- decoding
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def block_bounds(N: int, block: int):
    """[(start, stop)] of every block of `block` tokens; the last may be short."""
    return [(s, min(s + block, N)) for s in range(0, N, block)]


# ----------------------------------------------------------------- pooling
def pool_mean(X: np.ndarray, block: int) -> np.ndarray:
    """Mean of the rows of every block of X [N, d], over valid rows only."""
    return np.stack([X[s:e].mean(axis=0) for s, e in block_bounds(X.shape[0], block)])


# ------------------------------------------------------- compressed scores
def block_logits(Qbar: np.ndarray, Kbar: np.ndarray, scale: float) -> np.ndarray:
    """s[i, j] = scale * <Qbar_i, Kbar_j>."""
    return scale * (Qbar @ Kbar.T)


def row_softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# ------------------------------------------------------------- selection
def topk_size(k_frac: float, n_k: int) -> int:
    """K_k for a fraction k of n_k blocks (k as the float32 the ABI takes)."""
    kf = float(np.float32(k_frac))
    return min(n_k, max(1, math.ceil(kf * n_k - 1e-6)))


def selection_order(s: np.ndarray) -> np.ndarray:
    """Per row: block indices by score descending, equal scores by index ascending."""
    return np.argsort(-s, axis=-1, kind="stable")


def topp_size(P_sorted: np.ndarray, p_mass: float) -> np.ndarray:
    """m_p per row: the least m with sum of the first m sorted probabilities >= p.

    The cumulative sums are taken in fp64 in sorted order. p >= 1 keeps every
    block; if rounding keeps the total below p, every block is kept too.
    """
    p = float(np.float32(p_mass))
    rows, n_k = P_sorted.shape
    if p >= 1.0:
        return np.full(rows, n_k, dtype=np.int64)
    C = np.zeros((rows, n_k + 1))
    C[:, 1:] = np.cumsum(P_sorted, axis=1)
    reached = C >= p
    return np.where(reached.any(axis=1), reached.argmax(axis=1), n_k).astype(np.int64)


@dataclasses.dataclass
class RowSelection:
    kept: np.ndarray      # bool [rows, n_k]
    count: np.ndarray     # int  [rows]
    K_k: int
    m_p: np.ndarray       # int  [rows]
    order: np.ndarray     # int  [rows, n_k]
    margin: np.ndarray    # float [rows]; near-tie rows have margin < 1e-5


def hybrid_select(s: np.ndarray, k_frac: float, p_mass: float) -> RowSelection:
    """Union of Top-k and Top-p for every row of block logits s [rows, n_k]."""
    rows, n_k = s.shape
    P = row_softmax(s)
    order = selection_order(s)
    s_sorted = np.take_along_axis(s, order, axis=1)
    P_sorted = np.take_along_axis(P, order, axis=1)
    K_k = topk_size(k_frac, n_k)
    m_p = topp_size(P_sorted, p_mass)
    count = np.maximum(K_k, m_p)
    kept = np.zeros((rows, n_k), dtype=bool)
    ranks = np.arange(n_k)[None, :]
    np.put_along_axis(kept, order, ranks < count[:, None], axis=1)

    # distance of each row from a different decision
    margin = np.full(rows, np.inf)
    inner = count < n_k
    r = np.nonzero(inner)[0]
    margin[r] = s_sorted[r, count[r] - 1] - s_sorted[r, count[r]]
    p = float(np.float32(p_mass))
    if p < 1.0:
        C = np.zeros((rows, n_k + 1))
        C[:, 1:] = np.cumsum(P_sorted, axis=1)
        decided = (m_p >= K_k) & (m_p >= 1)
        r = np.nonzero(decided)[0]
        g = np.minimum(np.abs(C[r, m_p[r]] - p), np.abs(p - C[r, m_p[r] - 1]))
        margin[r] = np.minimum(margin[r], g)
    return RowSelection(kept, count, K_k, m_p, order, margin)


@dataclasses.dataclass
class MaskResult:
    kept: np.ndarray      # bool [B, H, n_q, n_k]
    cnt: np.ndarray       # int  [B, H, n_q]
    logits: np.ndarray    # fp64 [B, H, n_q, n_k]
    margin: np.ndarray    # fp64 [B, H, n_q]
    K_k: int
    m_p: np.ndarray       # int  [B, H, n_q]


def predict_mask_head(q: np.ndarray, k: np.ndarray, block_q: int, block_k: int,
                      k_frac: float, p_mass: float, scale: float) -> tuple:
    """Mask of one head from float64 q, k [N, d]: (RowSelection, logits)."""
    s = block_logits(pool_mean(q, block_q), pool_mean(k, block_k), scale)
    return hybrid_select(s, k_frac, p_mass), s


def predict_mask(Qb: np.ndarray, Kb: np.ndarray, block_q: int, block_k: int,
                 k_frac: float, p_mass: float, scale: float) -> MaskResult:
    """Hybrid mask of every (batch, head) from bf16 bit arrays [B, H, N, d]."""
    B, H, N, _ = Qb.shape
    n_q, n_k = -(-N // block_q), -(-N // block_k)
    kept = np.zeros((B, H, n_q, n_k), bool)
    cnt = np.zeros((B, H, n_q), np.int64)
    logits = np.zeros((B, H, n_q, n_k))
    margin = np.zeros((B, H, n_q))
    m_p = np.zeros((B, H, n_q), np.int64)
    K_k = topk_size(k_frac, n_k)
    for b in range(B):
        for h in range(H):
            sel, s = predict_mask_head(bf16_to_f64(Qb[b, h]), bf16_to_f64(Kb[b, h]),
                                       block_q, block_k, k_frac, p_mass, scale)
            kept[b, h], cnt[b, h], logits[b, h] = sel.kept, sel.count, s
            margin[b, h], m_p[b, h] = sel.margin, sel.m_p
    return MaskResult(kept, cnt, logits, margin, K_k, m_p)


# ------------------------------------------------------------ SLA2 router
def router_project(Xbar: np.ndarray, W: np.ndarray) -> np.ndarray:
    """The router's learnable linear projection of pooled rows (SLA2 page,
    section 2B: proj_q, proj_k applied to the pooled Q and K): Xbar [n, d] @ W
    [d, d_out], W given as the float32 values of the weights."""
    return Xbar @ np.asarray(W, np.float32).astype(np.float64)


def predict_mask_routed_head(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray,
                             block_q: int, block_k: int, k_frac: float, p_mass: float,
                             scale: float) -> tuple:
    """Mask of one head whose compressed score is taken between the projected
    pooled queries and keys: s = scale * (Qbar Wq)(Kbar Wk)^T, then the hybrid
    selection as before (p = 0 gives the router's hard Top-k)."""
    s = block_logits(router_project(pool_mean(q, block_q), wq),
                     router_project(pool_mean(k, block_k), wk), scale)
    return hybrid_select(s, k_frac, p_mass), s


def predict_mask_routed(Qb: np.ndarray, Kb: np.ndarray, Wq: np.ndarray, Wk: np.ndarray,
                        block_q: int, block_k: int, k_frac: float, p_mass: float,
                        scale: float) -> MaskResult:
    """Routed mask of every (batch, head); Wq, Wk [H, d, d] float32 (per head)."""
    B, H, N, _ = Qb.shape
    n_q, n_k = -(-N // block_q), -(-N // block_k)
    kept = np.zeros((B, H, n_q, n_k), bool)
    cnt = np.zeros((B, H, n_q), np.int64)
    logits = np.zeros((B, H, n_q, n_k))
    margin = np.zeros((B, H, n_q))
    m_p = np.zeros((B, H, n_q), np.int64)
    K_k = topk_size(k_frac, n_k)
    for b in range(B):
        for h in range(H):
            sel, s = predict_mask_routed_head(bf16_to_f64(Qb[b, h]), bf16_to_f64(Kb[b, h]),
                                              Wq[h], Wk[h], block_q, block_k, k_frac, p_mass,
                                              scale)
            kept[b, h], cnt[b, h], logits[b, h] = sel.kept, sel.count, s
            margin[b, h], m_p[b, h] = sel.margin, sel.m_p
    return MaskResult(kept, cnt, logits, margin, K_k, m_p)


def kept_to_bits(kept: np.ndarray) -> np.ndarray:
    """bool [..., n_k] -> uint32 [..., ceil(n_k/32)]: bit j%32 of word j//32."""
    n_k = kept.shape[-1]
    words = -(-n_k // 32)
    out = np.zeros(kept.shape[:-1] + (words,), np.uint32)
    for j in range(n_k):
        out[..., j // 32] |= kept[..., j].astype(np.uint32) << np.uint32(j % 32)
    return out


def kept_to_index_list(kept: np.ndarray):
    """bool [..., n_k] -> (idx int32 [..., n_k] ascending then -1, cnt int32 [...])."""
    n_k = kept.shape[-1]
    flat = kept.reshape(-1, n_k)
    idx = np.full(flat.shape, -1, np.int32)
    cnt = flat.sum(axis=1).astype(np.int32)
    for r in range(flat.shape[0]):
        nz = np.nonzero(flat[r])[0]
        idx[r, : nz.size] = nz
    return idx.reshape(kept.shape), cnt.reshape(kept.shape[:-1])


# ------------------------------------------------------------- attention
def _kept_tokens(row_kept: np.ndarray, N: int, block_k: int) -> np.ndarray:
    bounds = block_bounds(N, block_k)
    parts = [np.arange(*bounds[j]) for j in np.nonzero(row_kept)[0]]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def masked_attention_head(q, k, v, kept, block_q: int, block_k: int, scale: float,
                          q_blocks=None) -> np.ndarray:
    """Softmax attention of one head with every dropped key block masked out.

    q, k, v: float64 [N, d]; kept: bool [n_q, n_k]. Returns float64 [N, d]
    (rows of query blocks not in `q_blocks` are left as NaN). A query block
    with no kept key block yields zeros.
    """
    N, d = q.shape
    out = np.full((N, v.shape[1]), np.nan)
    qb = block_bounds(N, block_q)
    for i in (range(len(qb)) if q_blocks is None else q_blocks):
        s0, s1 = qb[i]
        toks = _kept_tokens(kept[i], N, block_k)
        if toks.size == 0:
            out[s0:s1] = 0.0
            continue
        P = row_softmax(scale * (q[s0:s1] @ k[toks].T))
        out[s0:s1] = P @ v[toks]
    return out


def elu_plus_one(x: np.ndarray) -> np.ndarray:
    """phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_branch_head(q, k, v, kept, block_q: int, block_k: int,
                       q_blocks=None) -> np.ndarray:
    """Linear attention of every query over the keys of its dropped blocks.

    O_l[t] = sum_u (phi(q_t).phi(k_u)) v_u / sum_u phi(q_t).phi(k_u), u over
    the valid tokens of the blocks that row block(t) dropped; zero if none.
    """
    N, d = q.shape
    out = np.full((N, v.shape[1]), np.nan)
    qb = block_bounds(N, block_q)
    for i in (range(len(qb)) if q_blocks is None else q_blocks):
        s0, s1 = qb[i]
        toks = _kept_tokens(~kept[i], N, block_k)
        if toks.size == 0:
            out[s0:s1] = 0.0
            continue
        W = elu_plus_one(q[s0:s1]) @ elu_plus_one(k[toks]).T
        out[s0:s1] = (W @ v[toks]) / W.sum(axis=1, keepdims=True)
    return out


def sparse_linear_attention_head(q, k, v, kept, block_q: int, block_k: int,
                                 scale: float, alpha: float, q_blocks=None):
    """O = O_s + alpha * O_l for one head."""
    o_s = masked_attention_head(q, k, v, kept, block_q, block_k, scale, q_blocks)
    o_l = linear_branch_head(q, k, v, kept, block_q, block_k, q_blocks)
    return o_s + float(np.float32(alpha)) * o_l


def sla2_mix_attention_head(q, k, v, kept, block_q: int, block_k: int, scale: float,
                            alpha, q_blocks=None):
    """SLA2's faithful sparse-linear output for one head (SLA2 page, section 2A):
    O = alpha (*) O_s + (1 - alpha) (*) O_l, alpha [d] (float32 values in [0, 1],
    one per output channel, the same for every row); O_s the block-sparse
    softmax attention, O_l the elu + 1 linear attention over the dropped keys
    (zero when no block was dropped)."""
    o_s = masked_attention_head(q, k, v, kept, block_q, block_k, scale, q_blocks)
    o_l = linear_branch_head(q, k, v, kept, block_q, block_k, q_blocks)
    a = np.asarray(alpha, np.float32).astype(np.float64)
    return a * o_s + (1.0 - a) * o_l


# ----------------------------------------------------- SALAD branch dropping
def linear_branch_dropped(weights, tau: float) -> bool:
    """Post-tuning branch dropping (SALAD page): the linear branch of a head is
    removed when its scale is small. Reading: removed iff every weight it is
    multiplied by has magnitude <= tau; the weights and the comparison are
    taken in float32, so tau = 0 removes only a branch whose weights are all
    exactly zero, which changes no output value."""
    w = np.abs(np.asarray(weights, np.float32))
    return bool(np.max(w) <= np.float32(tau))


def linear_weights_of_mix(alpha) -> np.ndarray:
    """The per-channel weights of O_l in the SLA2 mix, 1 - alpha, in float32."""
    return np.float32(1.0) - np.asarray(alpha, np.float32)


def sparse_linear_attention_head_dropping(q, k, v, kept, block_q: int, block_k: int,
                                          scale: float, alpha: float, tau: float,
                                          q_blocks=None):
    """O = O_s + alpha * O_l, or O_s alone when the branch is dropped."""
    if linear_branch_dropped([alpha], tau):
        return masked_attention_head(q, k, v, kept, block_q, block_k, scale, q_blocks)
    return sparse_linear_attention_head(q, k, v, kept, block_q, block_k, scale, alpha, q_blocks)


def sla2_mix_attention_head_dropping(q, k, v, kept, block_q: int, block_k: int, scale: float,
                                     alpha, tau: float, q_blocks=None):
    """The SLA2 mix, or alpha (*) O_s alone when its linear term is dropped."""
    if linear_branch_dropped(linear_weights_of_mix(alpha), tau):
        a = np.asarray(alpha, np.float32).astype(np.float64)
        return a * masked_attention_head(q, k, v, kept, block_q, block_k, scale, q_blocks)
    return sla2_mix_attention_head(q, k, v, kept, block_q, block_k, scale, alpha, q_blocks)


# ------------------------------------------------- sparse attention backward
def masked_scores_head(q, k, kept, block_q: int, block_k: int, scale: float) -> np.ndarray:
    """scale * Q K^T with -inf wherever the key's block is dropped for the
    query's row block; float64 [N, N]."""
    N = q.shape[0]
    qb, kb = np.arange(N) // block_q, np.arange(N) // block_k
    s = scale * (q @ k.T)
    return np.where(kept[qb][:, kb], s, -np.inf)


def masked_attention_lse_head(q, k, kept, block_q: int, block_k: int, scale: float,
                              q_blocks=None) -> np.ndarray:
    """log sum_u exp(scale q_t . k_u) over the kept keys of each row t; -inf
    for a row with no kept key (the log of an empty sum); NaN for rows of
    query blocks not in `q_blocks`."""
    N = q.shape[0]
    out = np.full(N, np.nan)
    qb = block_bounds(N, block_q)
    for i in (range(len(qb)) if q_blocks is None else q_blocks):
        s0, s1 = qb[i]
        toks = _kept_tokens(kept[i], N, block_k)
        if toks.size == 0:
            out[s0:s1] = -np.inf
            continue
        s = scale * (q[s0:s1] @ k[toks].T)
        m = s.max(axis=1)
        out[s0:s1] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def masked_attention_backward_head(q, k, v, kept, block_q: int, block_k: int, scale: float,
                                   do: np.ndarray, o=None):
    """dQ, dK, dV of O = P V, P = softmax of the masked scores, for the
    upstream gradient dO (all float64 [N, d]). A row with no kept key has
    O = 0 and passes no gradient. With D_t = sum_c dO_tc O_tc:
        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
        dQ = scale dS K,  dK = scale dS^T Q.
    `o`, if given, is the output the backward is handed (for instance the
    forward's result rounded to bf16) and D is taken from it, as a backward
    that receives O does; by default O is the exact one."""
    s = masked_scores_head(q, k, kept, block_q, block_k, scale)
    m = s.max(axis=1, keepdims=True)
    live = np.isfinite(m[:, 0])
    P = np.zeros_like(s)
    e = np.exp(s[live] - m[live])
    P[live] = e / e.sum(axis=1, keepdims=True)
    o = P @ v if o is None else o
    dv = P.T @ do
    dp = do @ v.T
    D = (do * o).sum(axis=1, keepdims=True)
    ds = P * (dp - D)
    return scale * (ds @ k), scale * (ds.T @ q), dv


def masked_attention_backward_sampled(q, k, v, kept, block_q: int, block_k: int, scale: float,
                                      do: np.ndarray, q_blocks, k_blocks, o=None):
    """The same gradients as masked_attention_backward_head, evaluated only
    where sampled, row block by row block so that no N x N matrix is formed:
    dQ for the rows of `q_blocks`, dK and dV for the keys of `k_blocks` (every
    row block that keeps one of them contributes). Returns (dq, dk, dv) as
    float64 [N, d] with NaN outside the sampled rows / keys. `o` as for
    masked_attention_backward_head."""
    N, d = q.shape
    qb, kb = block_bounds(N, block_q), block_bounds(N, block_k)
    dq = np.full((N, d), np.nan)
    dk = np.full((N, d), np.nan)
    dv = np.full((N, d), np.nan)
    k_blocks = sorted(set(k_blocks))
    for j in k_blocks:
        dk[kb[j][0]:kb[j][1]] = 0.0
        dv[kb[j][0]:kb[j][1]] = 0.0
    rows = sorted(set(q_blocks) | {i for i in range(len(qb)) if kept[i, k_blocks].any()})
    for i in rows:
        s0, s1 = qb[i]
        toks = _kept_tokens(kept[i], N, block_k)
        if toks.size == 0:
            if i in q_blocks:
                dq[s0:s1] = 0.0
            continue
        P = row_softmax(scale * (q[s0:s1] @ k[toks].T))
        o_i = P @ v[toks] if o is None else o[s0:s1]
        D = (do[s0:s1] * o_i).sum(axis=1, keepdims=True)
        dS = P * (do[s0:s1] @ v[toks].T - D)
        if i in q_blocks:
            dq[s0:s1] = scale * (dS @ k[toks])
        for j in k_blocks:
            if not kept[i, j]:
                continue
            k0, k1 = kb[j]
            cols = np.searchsorted(toks, np.arange(k0, k1))  # kept tokens are ascending
            dk[k0:k1] += scale * (dS[:, cols].T @ q[s0:s1])
            dv[k0:k1] += P[:, cols].T @ do[s0:s1]
    return dq, dk, dv


# ------------------------------------------------ linear branch backward
def elu_plus_one_grad(x: np.ndarray) -> np.ndarray:
    """phi'(x) for phi = elu + 1: 1 for x > 0, exp(x) otherwise."""
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def linear_branch_backward_head(q, k, v, kept, block_q: int, block_k: int, g: np.ndarray):
    """dQ, dK, dV of the linear branch O_l (linear_branch_head) for an upstream
    gradient G on O_l (float64 [N, d]). Per row block i, with D_i its dropped
    keys, H = sum_{u in D_i} phi(K_u)^T V_u, z = sum_{u in D_i} phi(K_u) and for
    each of its rows num_t = phi(Q_t) H, den_t = phi(Q_t).z, O_l,t = num_t/den_t:
        dnum_t = G_t / den_t,   dden_t = -(G_t . O_l,t) / den_t,
        dphi(Q_t) = H dnum_t + z dden_t,
        dH = sum_t phi(Q_t)^T dnum_t,   dz = sum_t phi(Q_t) dden_t,
    and every dropped key u of the block receives dphi(K_u) += dH V_u + dz,
    dV_u += phi(K_u) dH; dQ, dK follow through phi'. A block that dropped
    nothing passes no gradient."""
    N, d = q.shape
    dq, dk, dv = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, v.shape[1]))
    fq, fk = elu_plus_one(q), elu_plus_one(k)
    dfk = np.zeros((N, d))
    for i, (s0, s1) in enumerate(block_bounds(N, block_q)):
        toks = _kept_tokens(~kept[i], N, block_k)
        if toks.size == 0:
            continue
        H = fk[toks].T @ v[toks]
        z = fk[toks].sum(axis=0)
        num = fq[s0:s1] @ H
        den = fq[s0:s1] @ z
        ol = num / den[:, None]
        dnum = g[s0:s1] / den[:, None]
        dden = -(g[s0:s1] * ol).sum(axis=1) / den
        dfq = dnum @ H.T + np.outer(dden, z)
        dq[s0:s1] = dfq * elu_plus_one_grad(q[s0:s1])
        dH = fq[s0:s1].T @ dnum
        dz = fq[s0:s1].T @ dden
        dfk[toks] += v[toks] @ dH.T + dz
        dv[toks] += fk[toks] @ dH
    dk = dfk * elu_plus_one_grad(k)
    return dq, dk, dv


def sparse_linear_attention_backward_head(q, k, v, kept, block_q: int, block_k: int,
                                          scale: float, alpha: float, do: np.ndarray, o=None):
    """dQ, dK, dV of O = O_s + alpha O_l: the sparse part receives dO (with
    D_t = dO_t . O_s,t, O_s = O - alpha O_l when the handed O is given), the
    linear part alpha dO."""
    o_s = None
    if o is not None:
        o_s = o - float(np.float32(alpha)) * linear_branch_head(q, k, v, kept, block_q, block_k)
    gs = masked_attention_backward_head(q, k, v, kept, block_q, block_k, scale, do, o=o_s)
    gl = linear_branch_backward_head(q, k, v, kept, block_q, block_k,
                                     float(np.float32(alpha)) * do)
    return tuple(a + b for a, b in zip(gs, gl))


def sla2_mix_attention_backward_head(q, k, v, kept, block_q: int, block_k: int, scale: float,
                                     alpha, do: np.ndarray, o=None):
    """dQ, dK, dV of O = alpha (*) O_s + (1 - alpha) (*) O_l: the sparse part
    receives alpha (*) dO (with O_s = (O - (1 - alpha) O_l) / alpha from a handed
    O, where alpha > 0), the linear part (1 - alpha) (*) dO."""
    a = np.asarray(alpha, np.float32).astype(np.float64)
    o_s = None
    if o is not None:
        o_s = (o - (1.0 - a) * linear_branch_head(q, k, v, kept, block_q, block_k)) / a
    gs = masked_attention_backward_head(q, k, v, kept, block_q, block_k, scale, a * do, o=o_s)
    gl = linear_branch_backward_head(q, k, v, kept, block_q, block_k, (1.0 - a) * do)
    return tuple(x + y for x, y in zip(gs, gl))


def linear_branch_backward_sampled(q, k, v, kept, block_q: int, block_k: int, g: np.ndarray,
                                   q_blocks, k_blocks):
    """linear_branch_backward_head evaluated only where sampled: dQ for the rows
    of `q_blocks`, dK and dV for the keys of `k_blocks` (every row block that
    drops one of them contributes). NaN elsewhere."""
    N, d = q.shape
    qb, kb = block_bounds(N, block_q), block_bounds(N, block_k)
    dq = np.full((N, d), np.nan)
    dk = np.full((N, d), np.nan)
    dv = np.full((N, v.shape[1]), np.nan)
    k_blocks = sorted(set(k_blocks))
    keys = np.concatenate([np.arange(*kb[j]) for j in k_blocks])
    dfk = np.zeros((keys.size, d))
    dvk = np.zeros((keys.size, v.shape[1]))
    fk = elu_plus_one(k)
    for i, (s0, s1) in enumerate(qb):
        drops = [j for j in k_blocks if not kept[i, j]]
        if i not in q_blocks and not drops:
            continue
        toks = _kept_tokens(~kept[i], N, block_k)
        if toks.size == 0:
            if i in q_blocks:
                dq[s0:s1] = 0.0
            continue
        fq = elu_plus_one(q[s0:s1])
        H = fk[toks].T @ v[toks]
        z = fk[toks].sum(axis=0)
        num, den = fq @ H, fq @ z
        ol = num / den[:, None]
        dnum = g[s0:s1] / den[:, None]
        dden = -(g[s0:s1] * ol).sum(axis=1) / den
        if i in q_blocks:
            dq[s0:s1] = (dnum @ H.T + np.outer(dden, z)) * elu_plus_one_grad(q[s0:s1])
        if drops:
            dH = fq.T @ dnum
            dz = fq.T @ dden
            sel = np.isin(keys, np.concatenate([np.arange(*kb[j]) for j in drops]))
            dfk[sel] += v[keys[sel]] @ dH.T + dz
            dvk[sel] += fk[keys[sel]] @ dH
    dk[keys] = dfk * elu_plus_one_grad(k[keys])
    dv[keys] = dvk
    return dq, dk, dv


# --------------------------------------------------- low-bit sparse branch
# SLA2 page, section 2C: the sparse branch runs with Q, K, P and V quantised in
# the forward pass (low-bit attention such as INT8/FP8). Readings of what the
# page leaves open: Q and K as INT8 with one float32 scale per block (query
# blocks of block_q rows, key blocks of block_k rows): scale = amax / 127,
# code = round-half-even(x * (127 / amax)) taken in float32; V as FP8 e4m3
# (OCP e4m3fn: bias 7, largest finite 448) with one scale per (head, channel):
# code = e4m3(x * (448 / amax)) in float32; P as e4m3 codes of 448 p, with p
# taken against an exact running row maximum (so p <= 1), blocks visited in
# the order of the row's list; O = sum p~ v~ / sum p~ over the visited blocks.
E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an OCP e4m3fn byte (0x7f and 0xff are NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9                 # subnormal: m/8 * 2^-6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value, ties to the even code; |x| must not exceed 464
    (the half-way point above 448)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    assert np.all(a <= 464.0), "outside the e4m3 range"
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                      # subnormals share 2^-6's quantum
    quantum = 2.0 ** (e - 3)
    r = np.round(a / quantum) * quantum          # np.round: half to even
    return np.sign(x) * np.minimum(r, E4M3_MAX)


def int8_block_codes(x: np.ndarray, block: int):
    """Rows of x (float32 values) in blocks of `block`: codes (int) and the
    float32 scale of each block."""
    x = np.asarray(x, np.float32)
    n = x.shape[0]
    codes = np.zeros(x.shape, np.int64)
    scales = []
    for s0, s1 in block_bounds(n, block):
        amax = np.float32(np.abs(x[s0:s1]).max())
        if amax == 0:
            scales.append(np.float32(0))
            continue
        inv = np.float32(127) / amax
        codes[s0:s1] = np.clip(np.rint(x[s0:s1] * inv), -127, 127).astype(np.int64)
        scales.append(amax / np.float32(127))
    return codes, np.array(scales, np.float32)


def e4m3_channel_codes(x: np.ndarray):
    """Columns of x (float32 values): e4m3 values of x * (448 / amax_c) and the
    float32 scale amax_c / 448 of each column."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=0).astype(np.float32)
    inv = np.where(amax > 0, np.float32(E4M3_MAX) / np.where(amax > 0, amax, 1), 0)
    vals = e4m3_round((x * inv.astype(np.float32)).astype(np.float32))
    return vals, (amax / np.float32(E4M3_MAX)).astype(np.float32)


def lowbit_attention_head(q, k, v, idx_rows, cnt_rows, block_q: int, block_k: int,
                          scale: float, q_blocks=None) -> np.ndarray:
    """The low-bit sparse branch for one head; q, k, v float64 [N, d] (bf16
    values), idx_rows/cnt_rows the row lists. Rows of blocks not in
    `q_blocks` are NaN; an empty list gives zeros."""
    N, d = q.shape
    qc, qs = int8_block_codes(q, block_q)
    kc, ks = int8_block_codes(k, block_k)
    vv, vs = e4m3_channel_codes(v)
    v_deq = vv * vs.astype(np.float64)           # dequantised V
    out = np.full((N, d), np.nan)
    kb = block_bounds(N, block_k)
    for i, (s0, s1) in enumerate(block_bounds(N, block_q)):
        if q_blocks is not None and i not in q_blocks:
            continue
        m = np.full(s1 - s0, -np.inf)
        l = np.zeros(s1 - s0)
        acc = np.zeros((s1 - s0, d))
        for e in range(int(cnt_rows[i])):
            j = int(idx_rows[i, e])
            k0, k1 = kb[j]
            dot = (qc[s0:s1] @ kc[k0:k1].T).astype(np.float32)      # exact integers
            s = dot * np.float32(qs[i] * ks[j])                      # float32, as stored
            m_new = np.maximum(m, s.max(axis=1).astype(np.float64))
            f = np.exp(scale * (m - m_new))
            f[np.isneginf(m)] = 0.0
            acc *= f[:, None]
            l *= f
            m = m_new
            p = np.exp(scale * (s.astype(np.float64) - m[:, None]))
            p8 = e4m3_round((p * E4M3_MAX).astype(np.float32)) / E4M3_MAX
            l += p8.sum(axis=1)
            acc += p8 @ v_deq[k0:k1]
        out[s0:s1] = acc / l[:, None] if cnt_rows[i] > 0 else 0.0
    return out


# ------------------------------------------------- SVG2 semantic permutation
# "Sparse VideoGen2" page, section 2A: Q and K tokens are clustered
# independently by k-means into C_q and C_k clusters and permuted so that each
# cluster is contiguous (the output is permuted back, so attention itself is
# unchanged); section 2B: scores between cluster centroids stand in for the
# attention scores, clusters are sorted by them and taken in order until the
# cumulative score reaches p. Readings of what the page leaves open: Lloyd's
# k-means with the initial centroids at tokens floor(c N / C), a fixed number
# of iterations, squared Euclidean distance in float64 with ties to the lower
# cluster, an empty cluster keeping its centroid, centroids the float64 mean of
# their members summed in token order; the centroid score has the attention's
# scale, and a key cluster's probability is weighted by its size (softmax of
# s + ln |cluster|, empty clusters excluded), so that a cluster stands for its
# tokens; the selection is the hybrid rule with Top-k reduced to one cluster.
def kmeans_assign(x: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """argmin_c |x - c|^2 per row (float64), ties to the lower c: computed as
    |c|^2 - 2 x.c, the part that depends on c."""
    d2 = (cent * cent).sum(axis=1)[None, :] - 2.0 * (x @ cent.T)
    return np.argmin(d2, axis=1)


def kmeans_update(x: np.ndarray, assign: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Mean of each cluster's members, summed in token order; an empty
    cluster keeps its centroid."""
    new = cent.copy()
    for c in range(cent.shape[0]):
        members = np.nonzero(assign == c)[0]
        if members.size:
            new[c] = np.cumsum(x[members], axis=0)[-1] / members.size
    return new


def kmeans(x: np.ndarray, n_clusters: int, iters: int):
    """Lloyd's k-means on the rows of x (float64): `iters` rounds of assign then
    update from centroids at rows floor(c N / C), then a final assignment.
    Returns (assignment, centroids)."""
    N = x.shape[0]
    cent = x[(np.arange(n_clusters) * N) // n_clusters].copy()
    for _ in range(iters):
        cent = kmeans_update(x, kmeans_assign(x, cent), cent)
    return kmeans_assign(x, cent), cent


def svg2_permutation(assign: np.ndarray, n_clusters: int):
    """Tokens ordered by cluster, in token order within a cluster: the
    permutation (position -> token) and each cluster's [start, end)."""
    perm = np.argsort(assign * len(assign) + np.arange(len(assign)), kind="stable")
    sizes = np.bincount(assign, minlength=n_clusters)
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    return perm, starts, sizes


def svg2_select(cq: np.ndarray, ck: np.ndarray, k_sizes: np.ndarray, scale: float,
                p_mass: float) -> RowSelection:
    """Top-p over key clusters for every query cluster on the size-weighted
    centroid scores (Top-k reduced to one cluster)."""
    s = scale * (cq @ ck.T)
    with np.errstate(divide="ignore"):
        s = s + np.log(k_sizes.astype(np.float64))[None, :]   # -inf for empty clusters
    return hybrid_select(s, 1.0 / len(k_sizes), p_mass), s


def svg2_attention_head(q, k, v, n_q_clusters: int, n_k_clusters: int, iters: int,
                        scale: float, p_mass: float, q_rows=None):
    """SVG2's sparse attention for one head (float64 [N, d] inputs): each query
    attends to the tokens of the key clusters its cluster selected. Returns
    (O, q-assignment, k-assignment, selection); with `q_rows`, O holds only
    those rows (in that order)."""
    qa, cq = kmeans(q, n_q_clusters, iters)
    ka, ck = kmeans(k, n_k_clusters, iters)
    sizes = np.bincount(ka, minlength=n_k_clusters)
    sel, _ = svg2_select(cq, ck, sizes, scale, p_mass)
    rows = np.arange(q.shape[0]) if q_rows is None else np.asarray(q_rows)
    mask = sel.kept[qa[rows]][:, ka]                             # token pairs
    s = np.where(mask, scale * (q[rows] @ k.T), -np.inf)
    P = np.exp(s - s.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    return P @ v, qa, ka, sel
