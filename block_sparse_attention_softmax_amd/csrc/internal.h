// Internal declarations shared by the HIP translation units of libsparge.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sparge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bit pattern, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// INT8 codes of the four bf16 values in w0, w1 (low half first) at
// inv = 127 / amax: rint(x * inv) in float32, clamped to [-127, 127], packed
// little-endian (the low-bit branch's Q and K codes).
__device__ __forceinline__ uint32_t int8_pack4(uint32_t w0, uint32_t w1, float inv) {
  const uint32_t ws[2] = {w0, w1};
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int lo = (int)fminf(fmaxf(rintf(bf16_lo(ws[e]) * inv), -127.0f), 127.0f);
    const int hi = (int)fminf(fmaxf(rintf(bf16_hi(ws[e]) * inv), -127.0f), 127.0f);
    word |= ((uint32_t)(lo & 0xFF) | ((uint32_t)(hi & 0xFF) << 8)) << (16 * e);
  }
  return word;
}

// Workgroup id -> tile id such that the tiles of one XCD are contiguous.
// Workgroups are dispatched round-robin over the 8 XCDs (wg % 8), so the
// remap gives each XCD a contiguous, head-major range of tiles and the
// query blocks of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int XCDS = 8;
  const int per = total / XCDS, rem = total % XCDS;
  const int x = wg % XCDS, pos = wg / XCDS;
  const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + pos;
}

// ---- launchers (each returns the hipError_t of its launches) ----
struct MaskLaunch {
  int phase;  // 0: the whole mask; 1: pooling only; 2: everything after the pooling
  // optional (pooling): INT8 codes and per-block scales of Q and K for the
  // low-bit branch, written by the pooling pass from the same blocks
  int8_t* qc;
  int8_t* kc;
  float* qsc;
  float* ksc;
  const uint16_t* q;
  const uint16_t* k;
  int B, H, N, d, block_q, block_k, n_q, n_k, npad, words;
  int K_k;        // Top-k size
  int keep_all;   // p_mass >= 1
  double p;       // Top-p mass
  double scale;
  double* qbar;   // [B*H, n_q, d]
  double* kbar;   // [B*H, n_k, d]
  double* logits; // [B*H, n_q, n_k]
  // router (optional): scores between Qbar Wq and Kbar Wk
  const float* wq;  // [H, d, d] float32, row = input channel; nullptr: no router
  const float* wk;
  double* wqT;      // [B*H, d, d] float64, W transposed (row = output channel)
  double* wkT;
  double* qbar_p;   // [B*H, n_q, d] projected pooled queries
  double* kbar_p;   // [B*H, n_k, d]
  uint32_t* bits;
  int32_t* idx;
  int32_t* cnt;
};
hipError_t launch_mask(const MaskLaunch& a, hipStream_t s);
// sc * X Y^T per (b, h) in float64: X [BH][nx][d], Y [BH][ny][d] -> [BH][nx][ny]
hipError_t launch_scores_f64(const double* x, const double* y, double* out, int BH, int nx,
                             int ny, int d, double sc, hipStream_t st);
// the hybrid selection alone, on a.logits ([B*H*n_q][n_k]) into bits / idx / cnt
hipError_t launch_select_rows(const MaskLaunch& a, hipStream_t st);

struct AttnLaunch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* o;
  int B, H, N, d, block_q, n_q, n_k;
  float scale;
  // workspace: V packed key-contiguous per block, [B*H, n_k, d, 64]
  uint16_t* vt;
  float* lse;  // [B*H, N] natural log-sum-exp of each row's kept scores, or nullptr
  // linear branch (alpha == nullptr: plain sparse attention)
  const float* alpha;  // kLinAdd: [H]; kLinMix: [H, d]
  int lin_mode;        // LinMode
  float drop_below;    // a head whose linear weights are all <= this in magnitude skips the branch
  int32_t* lin_on;     // [H] 1 where the branch is evaluated
  int32_t* lin_lists;  // [2 + 2*B*H] counts, then the b*H + h with the branch on, then off
  uint16_t* hj;        // [B*H, n_k, 2, d*d + d] bf16 planes of H_j^T and z_j per key block
  uint32_t* mbits;     // [B*H, n_q, ceil(n_k / 32)] bit j set where block j is dropped
  uint16_t* hd;        // [B*H, n_q, 2, d, d] bf16 planes of H_D^T per query block
  float* zd;           // [B*H, n_q, d] z_D per query block
};
constexpr int kLinMaxKeyBlocks = 4096;  // the linear forward's drop bitmaps (one LDS row each)
// how the linear branch meets the sparse output: O_s + alpha[h] O_l, or the
// per-channel mix alpha[h][c] O_s + (1 - alpha[h][c]) O_l
enum LinMode { kLinAdd = 0, kLinMix = 1 };
// pack (V, and phi(K) for the linear branch) then attend; or either half alone
enum AttnPhase { kPackAndAttend = 0, kPackOnly = 1, kAttendOnly = 2 };
hipError_t launch_attn(const AttnLaunch& a, hipStream_t s, AttnPhase phase = kPackAndAttend);
// backward of the block-sparse attention: dQ, dK, dV for an upstream dO
struct BwdLaunch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;  // [B*H, N] from the forward
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, H, N, d, block_q, n_q, n_k;
  float scale;
  unsigned char* workspace;  // bwd_workspace_bytes()
  // linear branch (alpha == nullptr: none), as in AttnLaunch; requires block_q == d
  const float* alpha;
  int lin_mode;
  float drop_below;
};
hipError_t launch_bwd(const BwdLaunch& a, hipStream_t s);
size_t bwd_workspace_bytes(int B, int H, int N, int d, int block_q, bool linear = false);
// low-bit sparse branch: INT8 Q, K per block, e4m3 V per channel, e4m3 P
struct LowbitLaunch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* o;
  int B, H, N, d, block_q, n_q, n_k;
  float scale;
  int phase;  // LowbitPhase
  // workspace (lowbit_layout)
  int8_t* qc;       // [B*H, N, d] INT8 codes of Q
  int8_t* kc;       // [B*H, N, d] INT8 codes of K
  float* qs;        // [B*H, n_q] scales of Q
  float* ks;        // [B*H, n_k] scales of K
  uint32_t* vmax;   // [B*H, d] amax of each V channel (float bits)
  uint8_t* vt8;     // [B*H, n_k, d, 64] e4m3 codes of V^T, packed
};
// everything from bf16 Q, K, V; only V's channel scales and packed codes; only
// the attention from codes already in the workspace
enum LowbitPhase { kLowbitAll = 0, kLowbitPackV = 1, kLowbitAttend = 2 };
hipError_t launch_lowbit(const LowbitLaunch& a, hipStream_t s);
size_t lowbit_workspace_bytes(int B, int H, int N, int d, int block_q);
void lowbit_layout(LowbitLaunch& a, unsigned char* workspace);
// SVG2: k-means permutation, centroid Top-p, attention over padded clusters
struct Svg2Launch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, H, N, d, block_q, Cq, Ck, iters;
  float scale;
  double p;
  int phase;  // Svg2Phase
  // per (b, h), upper bounds: padded query tiles; 16-key groups of the padded
  // keys; list entries of one query cluster (groups rounded up to whole
  // 64-key chunks); packed 64-slot V^T tiles
  int max_tiles, max_groups, max_list, n_ktiles;
  // workspace (svg2_layout)
  double *centq, *centk, *normq, *normk, *clog;
  // the assignment's bf16 filter: centroid planes, |c|^2 in float32, per (b, h)
  // cmax bits and listed-token counts (kaux), and the listed tokens
  uint16_t *chi, *clo;
  float* cnf;
  int32_t *kaux, *kflags;
  int32_t *assign_q, *assign_k, *rank, *ccount, *size_q, *size_k, *off_q, *off_k, *perm_q,
      *perm_k;
  uint32_t* sbits;
  int32_t *sidx, *scnt, *qpad_off, *kpad_off, *tile_cluster, *n_tiles, *tile_order, *lists,
      *list_cnt;
  uint16_t *qp, *kp, *vp, *vtp;
};
// everything; steps 1-3 and the gathers only; the attention only (from the workspace)
enum Svg2Phase { kSvg2All = 0, kSvg2Cluster = 1, kSvg2Attend = 2 };
hipError_t launch_svg2(const Svg2Launch& a, hipStream_t s);
// per (b, h) of a finished svg2 call: query-key token pairs that take part in
// the attention, and pairs the kernel computes (whole waves x whole chunks)
hipError_t launch_svg2_pairs(const Svg2Launch& a, unsigned long long* counts, hipStream_t s);
size_t svg2_workspace_bytes(int B, int H, int N, int d, int block_q, int Cq, int Ck);
size_t svg2_layout(Svg2Launch& a, unsigned char* workspace);  // fills pointers; returns bytes
size_t attn_workspace_bytes(int B, int H, int N, int d);    // packed V
size_t linear_workspace_bytes(int B, int H, int N, int d, int block_q);  // packed V + linear branch
// fills the linear branch's workspace pointers of a (w may be nullptr); returns bytes
size_t linear_layout(AttnLaunch& a, unsigned char* w, int B, int H, int N, int d, int block_q);

}  // namespace sparge
