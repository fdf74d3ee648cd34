/*
 * sparge.h - C ABI of libsparge.so: hybrid Top-k + Top-p block-sparse
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the page "SpargeAttention2: Trainable
 * Sparse Attention via Hybrid Top-k+Top-p Masking and Distillation
 * Fine-Tuning": a per-row mask that is the union of a Top-k and a Top-p
 * selection (section 2A), applied at the level of blocks by a block-sparse
 * FlashAttention kernel that skips the masked tiles (section 2C). The scores
 * that pick the blocks come from mean-pooled queries and keys ("SLA2:
 * Sparse-Linear Attention with Learnable Routing and QAT", section 2B: the
 * router compresses Q and K by pooling adjacent tokens and scores the pooled
 * pairs, never V). The optional linear branch over the dropped blocks is the
 * sparse + linear split of the SLA2 page (section 1) with a static per-head
 * down-scaling of the linear part, as the SALAD page describes it.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Q, K, V and O are device pointers to contiguous bfloat16 tensors of
 *    shape [B, H, N, d] (row-major; d fastest), passed as raw 16-bit
 *    patterns. They must be 16-byte aligned. The caller owns every buffer;
 *    the library allocates nothing.
 *  - Blocks: query block i covers tokens [i*block_q, min((i+1)*block_q, N)),
 *    key block j covers [j*block_k, min((j+1)*block_k, N)). n_q =
 *    ceil(N/block_q), n_k = ceil(N/block_k). The last block may be short.
 *  - Supported shapes: d in {64, 128}; block_q in {64, 128}; block_k = 64;
 *    B, H, N >= 1; n_k <= 4096 for the mask (N <= 262144).
 *  - `stream` is a hipStream_t cast to void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns; outputs are
 *    valid once the stream reaches that point.
 *  - Return value: SPARGE_OK, or a negative sparge_status. Arguments are
 *    checked on the host before anything is enqueued; on a failed check
 *    nothing is launched and sparge_last_error() says why. A failed launch
 *    returns SPARGE_ERR_HIP. No call throws.
 *  - Calls are thread-safe; the library keeps no state besides the
 *    per-thread error message and, per device, whether the dynamic-LDS
 *    limits of the mask-selection kernels have been raised: the first call
 *    on a device that selects a mask (sparge_mask_predict, _select,
 *    _predict_routed, svg2_attn_fwd), whatever its shape, raises them for
 *    every row width at once.
 *  - A call enqueues kernel launches only: no allocation, no memset, no copy
 *    and no synchronisation, so a sequence of calls may be captured into a
 *    HIP graph and replayed. Make one mask-selecting call (any shape) on the
 *    device before a capture, so that the one-time attribute change above
 *    is not made while capturing. A replay reads and writes the buffers
 *    given at capture.
 */
#ifndef SPARGE_H
#define SPARGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARGE_OK = 0,
  SPARGE_ERR_INVALID_ARG = -1, /* a bad size, value, pointer or workspace  */
  SPARGE_ERR_UNSUPPORTED = -2, /* valid request outside the built shapes   */
  SPARGE_ERR_HIP = -3          /* the HIP runtime reported an error        */
} sparge_status;

/* Device workspace (bytes) that sparge_mask_predict needs: the pooled
 * queries and keys and the block scores, all float64. Returns 0 for
 * arguments that sparge_mask_predict would reject. */
size_t sparge_mask_workspace_bytes(int B, int H, int N, int d, int block_q,
                                   int block_k);

/* Block mask by the hybrid Top-k + Top-p rule (SpargeAttention2 page,
 * sections 1 and 2A; pooled scores as on the SLA2 page, section 2B).
 *
 * For every (b, h) and query block i:
 *   Qbar_i, Kbar_j = means of the valid rows of query block i / key block j;
 *   s_ij  = scale * <Qbar_i, Kbar_j>, P_i = softmax over j of s_i;
 *   order = key blocks by s_ij descending, equal scores by lower j first;
 *   K_k   = min(n_k, max(1, ceil(k_frac * n_k - 1e-6)))   (Top-k size);
 *   m_p   = least m with P mass of the first m blocks >= p_mass, summed in
 *           that order (Top-p size); n_k if p_mass >= 1 or never reached;
 *   kept  = the first max(K_k, m_p) blocks of the order (the union of the
 *           Top-k and the Top-p sets, both prefixes of one order).
 * Pooling, scores, softmax and prefix sums are evaluated in float64.
 *
 *  q, k        : bf16 [B, H, N, d], device, 16-byte aligned.
 *  k_frac      : Top-k fraction, 0 < k_frac <= 1.
 *  p_mass      : Top-p mass, p_mass >= 0 (0 = Top-k alone; >= 1 = keep all).
 *  scale       : score scale, finite and > 0 (normally 1/sqrt(d)).
 *  mask_bits   : out uint32 [B, H, n_q, ceil(n_k/32)]; bit j%32 of word
 *                j/32 is set iff key block j is kept. 4-byte aligned.
 *  kv_idx      : out int32 [B, H, n_q, n_k]; the first kv_cnt entries of a
 *                row list the kept key blocks in ascending order; the rest
 *                of the row is left untouched. 4-byte aligned.
 *  kv_cnt      : out int32 [B, H, n_q], number of kept blocks per row.
 *  block_logits: optional out float64 [B, H, n_q, n_k] (the scores s), or
 *                NULL. 8-byte aligned.
 *  workspace   : device scratch of at least sparge_mask_workspace_bytes(),
 *                16-byte aligned; contents on entry do not matter. With
 *                block_logits given, the scores go there and the workspace
 *                needs only the pooled means (B*H*(n_q + n_k)*d*8 bytes, each
 *                part rounded up to 256).
 */
int sparge_mask_predict(const void* q, const void* k, int B, int H, int N, int d,
                        int block_q, int block_k, float k_frac, float p_mass,
                        float scale, uint32_t* mask_bits, int32_t* kv_idx,
                        int32_t* kv_cnt, double* block_logits, void* workspace,
                        size_t workspace_bytes, void* stream);

/* sparge_mask_predict for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace and allocates nothing (no hipMalloc,
 * hipFree or allocating library call); its scratch (the float64 pooled means
 * and, when block_logits is NULL, the float64 block scores) is one
 * library-owned device array of sparge_mask_noalloc_scratch_bytes() (64 MiB)
 * per GPU, held from the library's first use on that GPU until the process
 * ends. Shapes whose scratch exceeds it are rejected with
 * SPARGE_ERR_UNSUPPORTED before anything is enqueued (the Wan-1.3B shape
 * needs 22 MB; passing block_logits leaves only the means, B*H*(n_q + n_k)*d*8
 * bytes). Every call on a GPU shares that GPU's array, so calls that overlap
 * on one GPU (other streams, other threads) race on it: order them on one
 * stream or serialise them. Nothing in the array needs to start cleared.
 * The first call on a device also looks up the array's address there.
 * Arguments, outputs and results are those of sparge_mask_predict, bit for
 * bit. */
size_t sparge_mask_noalloc_scratch_bytes(void);
int sparge_mask_predict_noalloc(const void* q, const void* k, int B, int H, int N, int d,
                                int block_q, int block_k, float k_frac, float p_mass,
                                float scale, uint32_t* mask_bits, int32_t* kv_idx,
                                int32_t* kv_cnt, double* block_logits, void* stream);

/* The two halves of sparge_mask_predict, for callers that run other work
 * beside the second: sparge_mask_pool writes the pooled queries and keys
 * (Qbar, Kbar above) into the workspace; sparge_mask_select forms the block
 * scores from them and selects. Enqueued in that order on one stream, with
 * the same B, H, N, d, block sizes and workspace (its contents left alone in
 * between), they give exactly the outputs of one sparge_mask_predict call.
 * sparge_mask_pool reads only q and k (bandwidth-bound); sparge_mask_select
 * reads only the workspace. Arguments, layouts and errors as for
 * sparge_mask_predict; each checks the arguments it takes. */
int sparge_mask_pool(const void* q, const void* k, int B, int H, int N, int d, int block_q,
                     int block_k, void* workspace, size_t workspace_bytes, void* stream);
int sparge_mask_select(int B, int H, int N, int d, int block_q, int block_k, float k_frac,
                       float p_mass, float scale, uint32_t* mask_bits, int32_t* kv_idx,
                       int32_t* kv_cnt, double* block_logits, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Device workspace (bytes) of sparge_mask_predict_routed: that of
 * sparge_mask_predict plus the router weights as float64 and the projected
 * pooled queries and keys. Returns 0 for arguments it would reject. */
size_t sparge_mask_routed_workspace_bytes(int B, int H, int N, int d, int block_q,
                                          int block_k);

/* Block mask whose compressed score goes through a router, as in "SLA2:
 * Sparse-Linear Attention with Learnable Routing and QAT", section 2B: the
 * pooled queries and keys are projected by learnable linear maps before the
 * score, s_ij = scale * <Qbar_i W_q[h], Kbar_j W_k[h]>; the selection that
 * follows is the hybrid rule of sparge_mask_predict (p_mass = 0 gives the
 * router's hard Top-k, section 2D). Projections and scores are float64.
 *
 *  w_q, w_k : float32 [H, d, d], device, 4-byte aligned; per head, row c =
 *             input channel, column j = output channel (Xbar W).
 *  workspace: at least sparge_mask_routed_workspace_bytes(), 16-byte aligned.
 *  Other arguments and outputs as for sparge_mask_predict.
 */
int sparge_mask_predict_routed(const void* q, const void* k, const float* w_q,
                               const float* w_k, int B, int H, int N, int d, int block_q,
                               int block_k, float k_frac, float p_mass, float scale,
                               uint32_t* mask_bits, int32_t* kv_idx, int32_t* kv_cnt,
                               double* block_logits, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Device workspace (bytes) that sparge_attn_fwd needs: V re-packed per
 * 64-key block into key-contiguous rows (bf16, B*H*ceil(N/64)*64*d values).
 * Returns 0 for arguments that sparge_attn_fwd would reject. */
size_t sparge_attn_workspace_bytes(int B, int H, int N, int d);

/* Block-sparse attention forward (SpargeAttention2 page, section 2C): for
 * every query t of query block i,
 *   O_t = sum_u softmax_u(scale * <Q_t, K_u>) V_u
 * where u runs over the valid keys of the key blocks listed in row i of
 * kv_idx / kv_cnt only; blocks not listed are skipped entirely. A row with
 * kv_cnt = 0 yields zeros. Products use bf16 inputs with float32
 * accumulation; the softmax runs online in float32; O is rounded to bf16
 * (nearest even).
 *
 *  q, k, v   : bf16 [B, H, N, d], device, 16-byte aligned.
 *  kv_idx    : int32 [B, H, n_q, n_k]; first kv_cnt entries of each row are
 *              key block indices in [0, n_k). Any such list is accepted (for
 *              example the output of sparge_mask_predict, or a fixed local
 *              window), in any order; a block listed twice is attended twice.
 *              Counts are clamped to [0, n_k] and indices to [0, n_k - 1], so
 *              a corrupt list cannot read out of bounds.
 *  kv_cnt    : int32 [B, H, n_q].
 *  o         : out bf16 [B, H, N, d], device, 16-byte aligned; must not
 *              overlap the inputs.
 *  workspace : device scratch of at least sparge_attn_workspace_bytes(),
 *              16-byte aligned; contents on entry do not matter.
 */
int sparge_attn_fwd(const void* q, const void* k, const void* v,
                    const int32_t* kv_idx, const int32_t* kv_cnt, int B, int H,
                    int N, int d, int block_q, int block_k, float scale, void* o,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The two halves of sparge_attn_fwd, for callers that pack V once and attend
 * several times (different query sets or lists over the same K and V), or
 * that pack V on another stream while sparge_mask_predict runs (the mask
 * reads only Q and K). sparge_attn_fwd(...) == sparge_attn_pack(v, ...)
 * followed by sparge_attn_fwd_packed(...) on one stream, bit for bit.
 *
 * sparge_attn_pack writes the packed V into `workspace` (at least
 * sparge_attn_workspace_bytes(B, H, N, d), 16-byte aligned). v: bf16
 * [B, H, N, d], device, 16-byte aligned.
 *
 * sparge_attn_fwd_packed reads that workspace (it must hold the pack of the
 * V that goes with q and k, and must not be modified while the call runs);
 * other arguments as for sparge_attn_fwd. */
int sparge_attn_pack(const void* v, int B, int H, int N, int d, void* workspace,
                     size_t workspace_bytes, void* stream);
int sparge_attn_fwd_packed(const void* q, const void* k, const int32_t* kv_idx,
                           const int32_t* kv_cnt, int B, int H, int N, int d,
                           int block_q, int block_k, float scale, void* o,
                           const void* workspace, size_t workspace_bytes, void* stream);

/* sparge_attn_fwd that also stores, for the backward, the natural
 * log-sum-exp of every row's kept scores:
 *   lse[b][h][t] = ln sum_{u kept for t} exp(scale * Q_t . K_u),
 * -inf for a row whose list is empty. Computed from the forward's own float32
 * running maximum and sum (the sum of the bf16-rounded weights it normalises
 * by). O is bit for bit that of sparge_attn_fwd.
 *
 *  lse : out float32 [B, H, N], device, 4-byte aligned.
 *  Other arguments as for sparge_attn_fwd. */
int sparge_attn_fwd_lse(const void* q, const void* k, const void* v,
                        const int32_t* kv_idx, const int32_t* kv_cnt, int B, int H, int N,
                        int d, int block_q, int block_k, float scale, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace (bytes) of sparge_attn_bwd: K packed like V (fp16), two
 * float32 values per row (rows padded to whole query blocks), and the
 * transposed lists (for every key block, the query blocks that list it):
 * about B*H*N*d*2 + 8*B*H*N + 8*B*H*n_q*n_k bytes. Returns 0 for arguments
 * sparge_attn_bwd would reject. */
size_t sparge_attn_bwd_workspace_bytes(int B, int H, int N, int d, int block_q, int block_k);

/* Backward of sparge_attn_fwd (the sparse attention is fine-tuned in the
 * SpargeAttention2 page, section 2B). For O = P V with P the softmax over the
 * listed keys of scale Q K^T and an upstream gradient dO, with
 * D_t = dO_t . O_t:
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * P is recomputed in float32 as exp(scale Q_t.K_u - lse_t); products take
 * 16-bit operands with float32 accumulation: bf16 (P and dS rounded to
 * bf16), except dQ = scale dS K, which takes dS and K as fp16 (a row's dS
 * sums to zero, so dQ cancels where the kept keys are alike, and fp16 keeps
 * three more bits; K must lie within fp16's range, |K| <= 65504, a larger
 * value giving an infinite dQ, and values under 2^-14 keep fewer bits as fp16
 * subnormals); dQ, dK, dV
 * are rounded to bf16. The same kv_idx / kv_cnt as the forward (any
 * order; a block listed twice counts twice); keys in no list get dK = dV = 0,
 * rows with an empty list dQ = 0. Deterministic: no atomics on the results.
 *
 *  q, k, v, o, d_o : bf16 [B, H, N, d], device, 16-byte aligned (o and lse
 *                    from sparge_attn_fwd_lse on the same q, k, v and lists).
 *  lse             : float32 [B, H, N], device.
 *  dq, dk, dv      : out bf16 [B, H, N, d], device, 16-byte aligned; must
 *                    not overlap the inputs or each other.
 *  workspace       : device scratch of at least sparge_attn_bwd_workspace_bytes(),
 *                    16-byte aligned; contents on entry do not matter.
 *  Other arguments as for sparge_attn_fwd. */
int sparge_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                    const void* d_o, const float* lse, const int32_t* kv_idx,
                    const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                    int block_k, float scale, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Device workspace (bytes) of sparse_linear_attn_fwd: the packed V of
 * sparge_attn_fwd; per (b, h) and key block
 * the summary phi(K_j)^T V_j (d x d) and sum phi(K_j) (d) as two bf16 planes
 * (hi and the rounded remainder); per (b, h) the drop bits (one uint32 per
 * 32 key blocks, rounded up, per query block); per query block
 * the dropped-block sums as two bf16 planes of d x d and d float32; and
 * H + 2 + 2*B*H int32 for the per-head branch flags and the lists of
 * (batch, head) pairs by flag; each part rounded up to 256 bytes. Returns 0
 * for arguments that sparse_linear_attn_fwd would reject. */
size_t sparse_linear_workspace_bytes(int B, int H, int N, int d);

/* Sparse attention plus a linear-attention branch over the dropped blocks
 * (sparse / linear split of the SLA2 page, section 1; static down-scaling of
 * the linear branch as on the SALAD page):
 *   O_t = O_s,t + alpha[h] * O_l,t,
 * O_s as in sparge_attn_fwd, and with phi(x) = elu(x) + 1 elementwise and D_i
 * the valid keys of the blocks NOT listed in row i,
 *   O_l,t = sum_{u in D_i} (phi(Q_t).phi(K_u)) V_u / sum_{u in D_i} phi(Q_t).phi(K_u),
 * and O_l,t = 0 when D_i is empty. phi is applied to the unscaled Q and K.
 * The linear branch forms per-key-block sums in float32 from bf16-rounded
 * phi(K) and V, carries them and their sums over D_i with about 16
 * significant bits (two bf16 planes) and accumulates in float32; its final
 * product phi(Q) . (sum over D_i) carries about 16 significant bits per
 * operand. Built for block_q == d (64 or 128) and at most 4096 key blocks
 * (N <= 262144); other sizes return SPARGE_ERR_UNSUPPORTED.
 *
 * Post-tuning branch dropping (SALAD page): a head with |alpha[h]| <=
 * drop_below (float32 comparison) skips its linear branch entirely (no phi(K)
 * packing, summaries or H products) and its output is O_s alone. The decision
 * is taken on the device, so alpha may change between calls without a host
 * synchronisation. drop_below = 0 skips only heads with alpha[h] == 0, which
 * changes no output value; a negative or NaN drop_below skips none.
 *
 *  alpha     : float32 [H], device, 4-byte aligned.
 *  lse       : nullptr, or out float32 [B, H, N], device, 4-byte aligned: the
 *              log-sum-exp of each row's kept scores (of the sparse part), as
 *              sparge_attn_fwd_lse writes it, for sparse_linear_attn_bwd.
 *  workspace : device scratch of at least sparse_linear_workspace_bytes(),
 *              16-byte aligned; contents on entry do not matter.
 *  Other arguments as for sparge_attn_fwd. */
int sparse_linear_attn_fwd(const void* q, const void* k, const void* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt,
                           const float* alpha, int B, int H, int N, int d,
                           int block_q, int block_k, float scale, float drop_below,
                           void* o, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* SLA2's faithful sparse-linear output (SLA2 page, section 2A): a learned
 * vector alpha in [0, 1] weighs the two branches channel by channel,
 *   O_t[c] = alpha[h][c] * O_s,t[c] + (1 - alpha[h][c]) * O_l,t[c],
 * with O_s and O_l (zero when D_i is empty) as in sparse_linear_attn_fwd.
 * alpha holds one value per output channel of each head; a per-head ratio
 * is the case of equal channels. Branch dropping as in
 * sparse_linear_attn_fwd, on the weights 1 - alpha[h][c] (float32): a head
 * whose every |1 - alpha[h][c]| <= drop_below has output alpha[h][c] O_s,t[c].
 *
 *  alpha     : float32 [H, d] row-major, device, 16-byte aligned.
 *  workspace : as for sparse_linear_attn_fwd (same size).
 *  Other arguments (lse included) as for sparse_linear_attn_fwd. */
int sla2_mix_attn_fwd(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                      const int32_t* kv_cnt, const float* alpha, int B, int H, int N, int d,
                      int block_q, int block_k, float scale, float drop_below, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace (bytes) of sparge_attn_fwd_lowbit: INT8 codes of Q and K,
 * their per-block scales, the per-channel scales of V and its packed e4m3
 * codes (about 3 * B*H*N*d bytes). Returns 0 for arguments it would reject. */
size_t sparge_attn_lowbit_workspace_bytes(int B, int H, int N, int d, int block_q,
                                          int block_k);

/* The sparse branch with low-bit operands (SLA2 page, section 2C: Q, K, P and
 * V quantised in the forward pass), over the key blocks of kv_idx / kv_cnt:
 *   Q, K : INT8, one float32 scale per block (block_q query rows; 64 keys):
 *          scale = amax / 127, code = round-half-even(x * (127 / amax)) in float32;
 *   V    : FP8 e4m3 (OCP e4m3fn, largest 448), one scale per (b, h, channel):
 *          code = e4m3(x * (448 / amax_c)), round to nearest even;
 *   S    : exact integer dot products of the codes times (scale_q scale_k);
 *   P    : e4m3 codes of 448 exp(scale (S - m)), m the exact running row
 *          maximum over the blocks visited so far, in list order (P <= 1);
 *   O    = sum P~ V~ / sum P~ over the listed blocks, rounded to bf16
 *          (zeros for an empty list).
 * S^T runs on INT8 MFMA (v_mfma_i32_32x32x32_i8) and P V on FP8 MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales), float32 accumulation. The
 * result depends on the order of each row's list only through rounding.
 *
 *  workspace : at least sparge_attn_lowbit_workspace_bytes(), 256-byte
 *              aligned; contents on entry do not matter.
 *  Other arguments as for sparge_attn_fwd. */
int sparge_attn_fwd_lowbit(const void* q, const void* k, const void* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, int B, int H, int N,
                           int d, int block_q, int block_k, float scale, void* o,
                           void* workspace, size_t workspace_bytes, void* stream);

/* sparge_attn_fwd_lowbit in parts, so that Q and K are not read again for
 * their INT8 codes: the mask's pooling pass already streams every query and
 * key block, so it writes the codes and scales of those same blocks.
 *
 *  sparge_mask_pool_lowbit      : sparge_mask_pool, whose pass also writes the
 *                                 INT8 codes and per-block scales of Q and K
 *                                 (as defined for sparge_attn_fwd_lowbit)
 *                                 into lowbit_workspace;
 *  sparge_attn_lowbit_pack      : V's per-channel scales and its packed e4m3
 *                                 codes into lowbit_workspace (reads v only);
 *  sparge_attn_fwd_lowbit_packed: the attention of sparge_attn_fwd_lowbit from
 *                                 the codes in lowbit_workspace (reads no
 *                                 bf16 input).
 * Enqueued on one stream with the same shapes and workspaces (the pack may
 * come before or after the pooling; sparge_mask_select between the pooling
 * and the attention as usual), they give exactly the outputs of
 * sparge_mask_pool + sparge_mask_select + sparge_attn_fwd_lowbit.
 * lowbit_workspace: at least sparge_attn_lowbit_workspace_bytes(), 256-byte
 * aligned; other arguments as for the calls named above. The attention may
 * be repeated on one pack and one pooling (other lists, same inputs). */
int sparge_mask_pool_lowbit(const void* q, const void* k, int B, int H, int N, int d,
                            int block_q, int block_k, void* workspace, size_t workspace_bytes,
                            void* lowbit_workspace, size_t lowbit_workspace_bytes,
                            void* stream);
int sparge_attn_lowbit_pack(const void* v, int B, int H, int N, int d, int block_q,
                            void* lowbit_workspace, size_t lowbit_workspace_bytes,
                            void* stream);
int sparge_attn_fwd_lowbit_packed(const int32_t* kv_idx, const int32_t* kv_cnt, int B, int H,
                                  int N, int d, int block_q, int block_k, float scale, void* o,
                                  void* lowbit_workspace, size_t lowbit_workspace_bytes,
                                  void* stream);

/* Device workspace (bytes) of svg2_attn_fwd (the clustering, the selection,
 * the tile order and the padded permuted Q, K, V); 0 for arguments
 * svg2_attn_fwd would reject. */
size_t svg2_attn_workspace_bytes(int B, int H, int N, int d, int block_q, int n_q_clusters,
                                 int n_k_clusters);

/* SVG2's semantic-aware sparse attention ("Sparse VideoGen2" page, section 2),
 * per (b, h):
 *  1. k-means of the query tokens into n_q_clusters and of the key tokens into
 *     n_k_clusters (Lloyd: `iters` rounds from centroids at tokens
 *     floor(c N / C), squared Euclidean distance in float64 with ties to the
 *     lower cluster, centroids the float64 mean of their members, an empty
 *     cluster keeps its centroid; then a final assignment);
 *  2. the tokens are permuted so each cluster is contiguous (in token order
 *     inside a cluster);
 *  3. every query cluster keeps the key clusters chosen by the hybrid rule of
 *     sparge_mask_predict on the logits scale * c_q . c_k + ln |key cluster|
 *     (empty clusters -inf), with Top-p mass p_mass and Top-k of one cluster;
 *  4. every query attends (softmax over scale Q K^T in float32, bf16 products)
 *     to the tokens of its cluster's kept key clusters; the output is written
 *     at the tokens' original positions, so O is the attention of the
 *     original sequence under that token-level mask.
 * q, k, v, o: bf16 [B, H, N, d], device, 16-byte aligned; block_q (64 or 128)
 * is the query tile of the attention step; at most 4096 key clusters. The
 * workspace (256-byte aligned) holds every intermediate: the centroids (and
 * their bf16 planes for the assignment's filter), assignments, counting-sort
 * counts and permutations, the centroid scores and selection, the group
 * lists, the query tiles' order, and Q, K, V and the packed V^T gathered
 * into cluster-contiguous order (query clusters padded to whole block_q
 * tiles, key clusters only to whole 16-key groups; svg2_attn_workspace_bytes
 * gives the total). */
int svg2_attn_fwd(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                  int block_q, int n_q_clusters, int n_k_clusters, int iters, float p_mass,
                  float scale, void* o, void* workspace, size_t workspace_bytes, void* stream);

/* svg2_attn_fwd in two parts: svg2_attn_cluster takes steps 1-3 and gathers
 * Q, K, V into the workspace (o is not touched); svg2_attn_apply then runs
 * step 4 from the workspace alone (reads no q, k, v) and writes o. Enqueued
 * in that order on one stream with the same shapes, cluster counts and
 * workspace, they give exactly svg2_attn_fwd's output; svg2_attn_apply may
 * be repeated. Arguments and errors as for svg2_attn_fwd. */
int svg2_attn_cluster(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                      int block_q, int n_q_clusters, int n_k_clusters, int iters, float p_mass,
                      float scale, void* workspace, size_t workspace_bytes, void* stream);
int svg2_attn_apply(int B, int H, int N, int d, int block_q, int n_q_clusters, int n_k_clusters,
                    float scale, void* o, void* workspace, size_t workspace_bytes, void* stream);

/* After an svg2_attn_fwd call on this stream, with the same arguments and its
 * workspace untouched since: per (b, h), counts[2 (b H + h)] = the query-key
 * token pairs that take part in the attention (each query with every token of
 * its cluster's kept key clusters) and counts[2 (b H + h) + 1] = the pairs
 * the attention kernel evaluates (whole block_q query tiles times whole
 * 64-key chunks, padding included). counts: uint64 [B, H, 2], device,
 * 8-byte aligned. For reporting the padding share; reads the workspace only. */
int svg2_attn_pair_counts(int B, int H, int N, int d, int block_q, int n_q_clusters,
                          int n_k_clusters, uint64_t* counts, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Device workspace (bytes) of sparse_linear_attn_bwd and sla2_mix_attn_bwd:
 * that of sparge_attn_bwd, plus the linear branch's packed V, its per-key-
 * block summaries, drop bits and per-query-block H_D, z_D as the forward
 * keeps them, the scaled dO of the mix, float32 dQ, dK, dV of the branch, and
 * per query block dH_D, dz_D and per key block their sums over the query
 * blocks that dropped it (two bf16 planes each, z parts float32 for the
 * latter), with the transposed drop bits. Returns 0 for arguments those calls
 * would reject. */
size_t sparse_linear_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward of sparse_linear_attn_fwd (O = O_s + alpha[h] O_l) for an upstream
 * gradient dO. The sparse part is sparge_attn_bwd's with the upstream gradient
 * dO and D_t = dO_t . O_s,t (taken as dO_t . O_t - G_t . O_l,t); the linear
 * part receives G = alpha[h] dO. With num_t = phi(Q_t) H_D, den_t = phi(Q_t).z_D
 * (H_D = sum over the dropped keys D_i of phi(K_u)^T V_u, z_D = sum phi(K_u)):
 *   dnum = G / den,  dden = -(G . O_l) / den,  dQ_t += (H_D dnum + z_D dden) phi'(Q_t),
 *   dK_u += (dH V_u + dz) phi'(K_u),  dV_u += phi(K_u) dH  for u in D_i,
 * dH = sum_t phi(Q_t)^T dnum_t, dz = sum_t phi(Q_t) dden_t over the rows of the
 * block (the chain rule of the SLA2 page's sparse-linear output, section 1).
 * The linear part runs in float32 on the vector units from H_D, z_D as the
 * forward forms them; dH, dz of each query block are summed per key block on
 * the matrix cores in two bf16 planes (about 16 significant bits per term,
 * float32 accumulation). It is added to the sparse part's float32 results
 * before dQ, dK, dV are rounded to bf16. Heads dropped by the same
 * rule as the forward (|alpha[h]| <= drop_below) pass no linear gradient.
 * Built for block_q == d and at most 4096 key blocks; deterministic.
 *
 *  o, lse    : from sparse_linear_attn_fwd with the same inputs (lse its
 *              lse output).
 *  alpha     : float32 [H], device.
 *  workspace : at least sparse_linear_bwd_workspace_bytes(), 16-byte aligned.
 *  Other arguments as for sparge_attn_bwd. */
int sparse_linear_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, const int32_t* kv_idx,
                           const int32_t* kv_cnt, const float* alpha, int B, int H, int N,
                           int d, int block_q, int block_k, float scale, float drop_below,
                           void* dq, void* dk, void* dv, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Backward of sla2_mix_attn_fwd (O = alpha (*) O_s + (1 - alpha) (*) O_l, SLA2
 * page, section 2A): as sparse_linear_attn_bwd with the sparse part receiving
 * alpha (*) dO (rounded to bf16) and the linear part (1 - alpha) (*) dO.
 *  alpha : float32 [H, d], device, 16-byte aligned.
 *  Other arguments as for sparse_linear_attn_bwd (o, lse from sla2_mix_attn_fwd). */
int sla2_mix_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* d_o, const float* lse, const int32_t* kv_idx,
                      const int32_t* kv_cnt, const float* alpha, int B, int H, int N, int d,
                      int block_q, int block_k, float scale, float drop_below, void* dq,
                      void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Message for the last non-OK return on the calling thread ("" if none).
 * The pointer stays valid until the next library call on that thread. */
const char* sparge_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARGE_H */
