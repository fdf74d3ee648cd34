// Block mask of the hybrid Top-k + Top-p rule, three steps:
//
//   pool_mean_kernel    Qbar, Kbar = means of the valid rows of every block
//                       (pooled queries and keys as on the SLA2 page,
//                       section 2B; mean pooling of blocks as the Sparse
//                       VideoGen2 page, section 1, names it). HBM-bound: it
//                       reads Q and K once.
//   block_logits_kernel s = scale * Qbar Kbar^T per head, float64 on the
//                       matrix cores.
//   selection           per query-block row: softmax of s, sort of (score
//                       desc, index asc), float64 prefix sum for Top-p, union
//                       with Top-k (SpargeAttention2 page, sections 1 and 2A),
//                       then the bitmask and the ascending index list.
//                       hybrid_select_reg_kernel: rows of up to 2048 blocks,
//                       one wave per row, the sort in registers and lane
//                       shuffles; hybrid_select_kernel: one workgroup per row,
//                       the sort in LDS, for wider rows and for rows of more
//                       than 512 blocks when there are too few of them to
//                       fill the chip one wave each.
//
// Everything that decides the mask is float64, so the selection is the one a
// float64 evaluation of the definition gives, up to summation order.
#include <algorithm>
#include <mutex>

#include "internal.h"

namespace sparge {
namespace {

constexpr int kThreads = 256;

// ----------------------------------------------------------------- pooling
// One workgroup per block of Q (blockIdx.x < nq) or K (the rest); grid.y =
// B*H. Thread t owns 16-byte column chunk t % CH and rows t / CH + RSTEP*i.
// With Q8 the same pass also writes the low-bit branch's INT8 codes of the
// block and its scale amax / 127 (the block is in registers already): the
// codes and scales quant_int8_kernel would produce, bit for bit.
template <int D, bool Q8 = false>
__global__ __launch_bounds__(kThreads) void pool_mean_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, double* __restrict__ qbar,
    double* __restrict__ kbar, int N, int block_q, int block_k, int nq, int nk,
    int8_t* __restrict__ qc = nullptr, int8_t* __restrict__ kc = nullptr,
    float* __restrict__ qsc = nullptr, float* __restrict__ ksc = nullptr) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int RSTEP = kThreads / CH;   // rows handled per pass
  __shared__ double red[kThreads][9];    // +1 pad against bank conflicts
  __shared__ float amx[kThreads / 64];

  const bool isq = (int)blockIdx.x < nq;
  const int blk = isq ? blockIdx.x : blockIdx.x - nq;
  const int block = isq ? block_q : block_k;
  const int nblk = isq ? nq : nk;
  const uint16_t* x = isq ? q : k;
  double* out = isq ? qbar : kbar;
  const int bh = blockIdx.y, t = threadIdx.x;
  const int c = t % CH, r0 = t / CH;
  const int start = blk * block;
  const int rows = min(block, N - start);
  const uint4* src =
      reinterpret_cast<const uint4*>(x + ((size_t)bh * N + start) * D) + c;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  // at most 128 rows per block: up to 8 (D=128) or 4 (D=64) loads per thread
  constexpr int MAXIT = 128 / RSTEP;
  uint4 w[MAXIT];
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int r = r0 + RSTEP * i;
    w[i] = r < rows ? src[(size_t)r * CH] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_lo(ws[e]);
      acc[2 * e + 1] += (double)bf16_hi(ws[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[t][e] = acc[e];
  if constexpr (Q8) {  // block amax (rows past the block are zeros), then the codes
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXIT; ++i) {
      const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) a = fmaxf(a, fmaxf(fabsf(bf16_lo(ws[e])), fabsf(bf16_hi(ws[e]))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((t & 63) == 0) amx[t >> 6] = a;
  }
  __syncthreads();
  if (t < D) {
    const int cc = t / 8, e = t % 8;
    double s = 0.0;
    for (int r = 0; r < RSTEP; ++r) s += red[r * CH + cc][e];
    out[((size_t)bh * nblk + blk) * D + t] = s / (double)rows;
  }
  if constexpr (Q8) {
    float amax = amx[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) amax = fmaxf(amax, amx[i]);
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (t == 0) (isq ? qsc : ksc)[(size_t)bh * nblk + blk] = amax / 127.0f;
    int8_t* codes = (isq ? qc : kc) + ((size_t)bh * N + start) * D + 8 * c;
#pragma unroll
    for (int i = 0; i < MAXIT; ++i) {
      const int r = r0 + RSTEP * i;
      if (r < rows)
        *reinterpret_cast<uint2*>(codes + (size_t)r * D) =
            make_uint2(int8_pack4(w[i].x, w[i].y, inv), int8_pack4(w[i].z, w[i].w, inv));
    }
  }
}

// ------------------------------------------------------------ block scores
// s[bh][i][j] = scale * sum_c qbar[bh][i][c] * kbar[bh][j][c], float64 on the
// matrix cores (v_mfma_f64_16x16x4_f64: lane l supplies A[l&15][l>>4] and
// B[l>>4][l&15] and holds D[4e + (l>>4)][l&15], e = 0..3). One wave per
// 32 x 32 output tile (2 x 2 MFMA tiles); each lane's 16-byte loads of Qbar and
// Kbar rows feed two k-steps (the same c order on both sides). Rows and
// columns past n_q / n_k read a valid row and are not stored.
typedef double f64x4 __attribute__((ext_vector_type(4)));
template <int D>
__global__ __launch_bounds__(kThreads) void block_logits_kernel(
    const double* __restrict__ qbar, const double* __restrict__ kbar,
    double* __restrict__ s, int n_q, int n_k, int tq, int tk, int tiles, double scale) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (tile >= tiles) return;
  const int bh = tile / (tq * tk), rem = tile % (tq * tk);
  const int i0 = (rem / tk) * 32, j0 = (rem % tk) * 32;
  const int r = lane & 15, g = lane >> 4;
  const double* qa = qbar + ((size_t)bh * n_q + min(i0 + r, n_q - 1)) * D + 2 * g;
  const double* qb = qbar + ((size_t)bh * n_q + min(i0 + 16 + r, n_q - 1)) * D + 2 * g;
  const double* ka = kbar + ((size_t)bh * n_k + min(j0 + r, n_k - 1)) * D + 2 * g;
  const double* kb = kbar + ((size_t)bh * n_k + min(j0 + 16 + r, n_k - 1)) * D + 2 * g;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int c0 = 0; c0 < D; c0 += 8) {
    const double2 xa = *reinterpret_cast<const double2*>(qa + c0);
    const double2 xb = *reinterpret_cast<const double2*>(qb + c0);
    const double2 ya = *reinterpret_cast<const double2*>(ka + c0);
    const double2 yb = *reinterpret_cast<const double2*>(kb + c0);
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.x, ya.x, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.x, yb.x, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(xb.x, ya.x, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(xb.x, yb.x, acc[1][1], 0, 0, 0);
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.y, ya.y, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.y, yb.y, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(xb.y, ya.y, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(xb.y, yb.y, acc[1][1], 0, 0, 0);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 16 * a + 4 * e + g, j = j0 + 16 * b + r;
        if (i < n_q && j < n_k) s[((size_t)bh * n_q + i) * n_k + j] = scale * acc[a][b][e];
      }
}

// ----------------------------------------------------------- router weights
// The router's projection weights (SLA2 page, section 2B: proj_q, proj_k on
// the pooled queries and keys), float32 [H][d][d] with row = input channel,
// as float64 W^T for every (b, h): wt[bh][j][c] = W[h][c][j]. The projection
// Xbar W is then the same "rows of A against rows of B" product as the block
// scores and runs in block_logits_kernel with scale 1.
__global__ __launch_bounds__(kThreads) void router_weights_kernel(const float* __restrict__ w,
                                                                  double* __restrict__ wt,
                                                                  int H, int d) {
  const int bh = blockIdx.y, h = bh % H;
  const int dd = d * d;
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < dd; e += gridDim.x * kThreads) {
    const int j = e / d, c = e % d;
    wt[(size_t)bh * dd + e] = (double)w[(size_t)h * dd + (size_t)c * d + j];
  }
}

// ------------------------------------------------------- wave-level helpers
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// inclusive scan over the 64 lanes of a wave
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}
// make this wave's LDS writes visible to its other lanes
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ----------------------------------------------------------- selection
// LDS bytes of one row of the selection kernel with npad sorted entries
__host__ __device__ constexpr size_t select_lds_bytes(int npad) {
  return (((size_t)npad * (2 * sizeof(double) + sizeof(uint16_t)) + 128 * sizeof(uint32_t)) + 15) &
         ~(size_t)15;
}
// threads per row: one compare-exchange pair each per sorting stage, at most 256
__host__ __device__ constexpr int select_threads(int npad) { return npad / 2 < 256 ? (npad / 2 < 64 ? 64 : npad / 2) : 256; }

// One workgroup per query-block row. LDS: sv[npad] doubles (scores, sorted in
// place), ev[npad] doubles (exp(s - max) by original index), si[npad] uint16,
// wb[words] uint32. Wave 0 loads the row, forms the softmax terms, takes the
// Top-p prefix and emits the outputs; all waves sort. A sorting stage whose
// compare distance keeps every pair of a wave inside that wave's 128 entries
// needs only a wave-local fence; the others take a workgroup barrier.
template <int NPAD>
__global__ __launch_bounds__(256) void hybrid_select_kernel(
    const double* __restrict__ s, int rows, int n_k, int words, int K_k,
    int keep_all, double p, uint32_t* __restrict__ bits_out,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int npad = NPAD;
  constexpr int TH = select_threads(NPAD);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  double* sv = reinterpret_cast<double*>(smem);
  double* ev = sv + npad;
  uint16_t* si = reinterpret_cast<uint16_t*>(ev + npad);
  uint32_t* wb = reinterpret_cast<uint32_t*>(si + npad);
  __shared__ double tot_s;
  const size_t row = blockIdx.x;
  const double* srow = s + row * (size_t)n_k;

  // 1. load scores (padding with -inf past n_k); row maximum and exp sum (wave 0)
  if (wave == 0) {
    double mx = -INFINITY;
    for (int j = lane; j < npad; j += 64) {
      const double v = j < n_k ? srow[j] : -INFINITY;
      sv[j] = v;
      si[j] = (uint16_t)j;
      mx = fmax(mx, v);
    }
    for (int w = lane; w < words; w += 64) wb[w] = 0u;
    mx = wave_max(mx);
    double tot = 0.0;
    for (int j = lane; j < n_k; j += 64) {
      const double e = exp(sv[j] - mx);  // this lane wrote sv[j] itself
      ev[j] = e;
      tot += e;
    }
    tot = wave_sum(tot);
    if (lane == 0) tot_s = tot;
  }
  __syncthreads();

  // 2. bitonic sort: position 0 = highest score, equal scores lower index
  //    first. All (score, index) pairs are distinct, so the order is total.
  constexpr int PAIRS = NPAD / 2, C = PAIRS / TH > 0 ? PAIRS / TH : 1;
#pragma unroll 1
  for (int kk = 2; kk <= NPAD; kk <<= 1) {
#pragma unroll 1
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      double a[C], b[C];
      int ia[C], ib[C], ii[C];
#pragma unroll
      for (int u = 0; u < C; ++u) {
        const int pi = (wave * C + u) * 64 + lane;  // each wave owns 64*C consecutive pairs
        ii[u] = 2 * pi - (pi & (jj - 1));
        if (pi < PAIRS) {
          a[u] = sv[ii[u]];
          b[u] = sv[ii[u] + jj];
          ia[u] = si[ii[u]];
          ib[u] = si[ii[u] + jj];
        }
      }
#pragma unroll
      for (int u = 0; u < C; ++u) {
        const int pi = (wave * C + u) * 64 + lane, i = ii[u];
        if (pi < PAIRS) {
          const bool l_first = (b[u] > a[u]) || (b[u] == a[u] && ib[u] < ia[u]);
          if (l_first == ((i & kk) == 0)) {
            sv[i] = b[u]; sv[i + jj] = a[u];
            si[i] = (uint16_t)ib[u]; si[i + jj] = (uint16_t)ia[u];
          }
        }
      }
      // a wave's pairs cover its own 128*C consecutive entries whenever the
      // distance is at most 64*C, so between two such stages a wave-local
      // fence suffices
      const int jn = jj > 1 ? jj >> 1 : kk;  // next stage's distance
      if (jj <= 64 * C && jn <= 64 * C) wave_lds_sync();
      else __syncthreads();
    }
  }
  if (wave != 0) return;  // no barrier follows
  const double tot = tot_s;

  // 3. Top-p: cumulative probability in sorted order; first prefix >= p.
  //    Lane L owns sorted positions [L*per, (L+1)*per).
  int m_p = n_k;
  if (!keep_all) {
    if (p <= 0.0) {
      m_p = 0;
    } else {
      const int per = npad / 64 > 0 ? npad / 64 : 1;
      const int r0 = lane * per;
      double local = 0.0;
      for (int r = r0; r < r0 + per && r < n_k; ++r) local += ev[si[r]] / tot;
      double run = wave_incl_scan(local, lane) - local;
      int hit = INT32_MAX;
      for (int r = r0; r < r0 + per && r < n_k; ++r) {
        run += ev[si[r]] / tot;
        if (run >= p) { hit = r + 1; break; }
      }
      const unsigned long long any = __ballot(hit != INT32_MAX);
      if (any) m_p = __shfl(hit, __ffsll((long long)any) - 1);
    }
  }
  const int count = max(K_k, m_p);

  // 4. union = first `count` of the order -> bitmask
  for (int r = lane; r < count; r += 64) {
    const int j = si[r];
    if (j < n_k) atomicOr(&wb[j >> 5], 1u << (j & 31));  // (only non-finite scores reach j >= n_k)
  }
  wave_lds_sync();

  // 5. emit bitmask, ascending index list and count (words <= 128: two per lane)
  const uint32_t w0 = lane < words ? wb[lane] : 0u;
  const uint32_t w1 = lane + 64 < words ? wb[lane + 64] : 0u;
  if (lane < words) bits_out[row * words + lane] = w0;
  if (lane + 64 < words) bits_out[row * words + lane + 64] = w1;
  const int c0 = __popc(w0), c1 = __popc(w1);
  const int e0 = wave_incl_scan(c0, lane) - c0;
  const int e1 = wave_sum(c0) + wave_incl_scan(c1, lane) - c1;
  int32_t* irow = idx_out + row * (size_t)n_k;
  uint32_t word = w0;
  int pos = e0;
  while (word) {
    irow[pos++] = lane * 32 + __ffs(word) - 1;
    word &= word - 1;
  }
  word = w1;
  pos = e1;
  while (word) {
    irow[pos++] = (lane + 64) * 32 + __ffs(word) - 1;
    word &= word - 1;
  }
  if (lane == 0) cnt_out[row] = count;
}

// Rows of up to 2048 padded entries: one wave per row, entries in registers.
// Lane L holds sorted positions L*E .. L*E+E-1 (E = NPAD/64) once the bitonic
// network has run; a compare distance below E pairs two registers of one
// lane, a larger one pairs the same register of lanes L and L ^ (jj/E),
// exchanged with shuffles. Up to 512 entries the whole network is unrolled;
// wider rows loop over the stages, with the in-lane distances (compile-time
// register pairs) unrolled per distance. The softmax total, the
// probabilities and the Top-p prefix sums are formed exactly as by the LDS
// variant above. With Top-k alone (p = 0) or p >= 1 the kept count is known
// before any ordering, so the kernel selects instead of sorting.
template <int NPAD>
__global__ __launch_bounds__(256) void hybrid_select_reg_kernel(
    const double* __restrict__ s, int rows, int n_k, int words, int K_k,
    int keep_all, double p, uint32_t* __restrict__ bits_out,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out) {
  constexpr int E = NPAD / 64;
  static_assert(E >= 1 && E <= 32, "register rows hold 64 .. 2048 entries");
  __shared__ uint32_t wbs[4][NPAD / 32 > 0 ? NPAD / 32 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wave;
  if (row >= (size_t)rows) return;  // whole wave leaves together
  uint32_t* wb = wbs[wave];
  const double* srow = s + row * (size_t)n_k;

  // 1. load (entry j = lane + 64e in register e), row maximum, exp sum in
  //    index order per lane
  double sc[E];
  int ix[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    sc[e] = j < n_k ? srow[j] : -INFINITY;
    ix[e] = j;
  }

  if (keep_all || !(p > 0.0)) {
    // Top-k alone (or every block): the count is known, and the kept set is
    // the `count` largest (score, index) pairs in the order above. No sort:
    // a bitwise search finds the count-th largest score key T, then the
    // entries scoring exactly T are taken in increasing index order.
    const int count = keep_all ? n_k : K_k;
    // order-preserving integer keys of the scores (-0 folded into +0 so
    // that equal scores get equal keys); entries past n_k get key 0, below
    // every score
    uint64_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t b = (uint64_t)__double_as_longlong(sc[e] + 0.0);
      key[e] = lane + 64 * e < n_k ? (b >> 63 ? ~b : b | (1ull << 63)) : 0ull;
    }
    uint64_t T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (c >= count) T = cand;
    }
    int ties = count;  // entries scoring T still to take
#pragma unroll
    for (int e = 0; e < E; ++e) ties -= __popcll(__ballot(key[e] > T));
    // emit in index order j = lane + 64 e: register by register, lanes in order
    const uint64_t below = (1ull << lane) - 1ull;
    int before = 0, pos = 0;
    uint32_t myword = 0u;
    int32_t* irow = idx_out + row * (size_t)n_k;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool eq = key[e] == T && key[e] != 0ull;
      const uint64_t meq = __ballot(eq);
      const bool kept = key[e] > T || (eq && before + __popcll(meq & below) < ties);
      before += __popcll(meq);
      const uint64_t mk = __ballot(kept);
      if (lane == 2 * e) myword = (uint32_t)mk;
      if (lane == 2 * e + 1) myword = (uint32_t)(mk >> 32);
      if (kept) irow[pos + __popcll(mk & below)] = lane + 64 * e;
      pos += __popcll(mk);
    }
    if (lane < words) bits_out[row * words + lane] = myword;
    if (lane == 0) cnt_out[row] = count;
    return;
  }

  for (int w = lane; w < words; w += 64) wb[w] = 0u;
  double mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) mx = fmax(mx, sc[e]);
  mx = wave_max(mx);
  double tot = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lane + 64 * e < n_k) tot += exp(sc[e] - mx);
  tot = wave_sum(tot);

  // 2. bitonic sort: position 0 = highest score, equal scores lower index first
  auto in_lane = [&](int jj, int kk) {  // jj < E: register pairs (e, e ^ jj)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e & jj) continue;
      const int f = e ^ jj;
      const bool desc = ((lane * E + e) & kk) == 0;
      const bool b_first = (sc[f] > sc[e]) || (sc[f] == sc[e] && ix[f] < ix[e]);
      if (b_first == desc) {
        const double ts = sc[e]; sc[e] = sc[f]; sc[f] = ts;
        const int ti = ix[e]; ix[e] = ix[f]; ix[f] = ti;
      }
    }
  };
  auto cross_lane = [&](int jj, int kk) {  // jj >= E: lanes L and L ^ (jj / E)
    const int m = jj / E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double os = __shfl_xor(sc[e], m);
      const int oi = __shfl_xor(ix[e], m);
      const int pos = lane * E + e;
      const bool lower = (pos & jj) == 0, desc = (pos & kk) == 0;
      const double as = lower ? sc[e] : os, bs = lower ? os : sc[e];
      const int ai = lower ? ix[e] : oi, bi = lower ? oi : ix[e];
      const bool b_first = (bs > as) || (bs == as && bi < ai);
      if (b_first == desc) { sc[e] = os; ix[e] = oi; }
    }
  };
  if constexpr (E <= 8) {
#pragma unroll
    for (int kk = 2; kk <= NPAD; kk <<= 1) {
#pragma unroll
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        if (jj < E) in_lane(jj, kk);
        else cross_lane(jj, kk);
      }
    }
  } else {
#pragma unroll 1
    for (int kk = 2; kk <= NPAD; kk <<= 1) {
#pragma unroll 1
      for (int jj = kk >> 1; jj >= E; jj >>= 1) cross_lane(jj, kk);
      // then the in-lane distances min(kk, E) / 2 .. 1, each unrolled
      const int jmax = min(kk, E) >> 1;
      if constexpr (E >= 32) if (jmax >= 16) in_lane(16, kk);
      if (jmax >= 8) in_lane(8, kk);
      if (jmax >= 4) in_lane(4, kk);
      if (jmax >= 2) in_lane(2, kk);
      in_lane(1, kk);
    }
  }

  // 3. Top-p: cumulative probability in sorted order; first prefix >= p
  int m_p = n_k;
  if (!keep_all) {
    if (p <= 0.0) {
      m_p = 0;
    } else {
      double pr[E];
#pragma unroll
      for (int e = 0; e < E; ++e) pr[e] = exp(sc[e] - mx) / tot;
      double local = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lane * E + e < n_k) local += pr[e];
      double run = wave_incl_scan(local, lane) - local;
      int hit = INT32_MAX;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lane * E + e < n_k && hit == INT32_MAX) {
          run += pr[e];
          if (run >= p) hit = lane * E + e + 1;
        }
      }
      const unsigned long long any = __ballot(hit != INT32_MAX);
      if (any) m_p = __shfl(hit, __ffsll((long long)any) - 1);
    }
  }
  const int count = max(K_k, m_p);

  // 4. union = first `count` of the order -> bitmask
  wave_lds_sync();  // wb cleared by every lane
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lane * E + e < count && ix[e] < n_k) atomicOr(&wb[ix[e] >> 5], 1u << (ix[e] & 31));
  wave_lds_sync();

  // 5. emit bitmask, ascending index list and count (words <= 64: one per lane)
  const uint32_t w0 = lane < words ? wb[lane] : 0u;
  if (lane < words) bits_out[row * words + lane] = w0;
  const int c0 = __popc(w0);
  const int e0 = wave_incl_scan(c0, lane) - c0;
  int32_t* irow = idx_out + row * (size_t)n_k;
  uint32_t word = w0;
  int pos = e0;
  while (word) {
    irow[pos++] = lane * 32 + __ffs(word) - 1;
    word &= word - 1;
  }
  if (lane == 0) cnt_out[row] = count;
}

template <int NPAD>
hipError_t launch_select_reg(const MaskLaunch& a, hipStream_t st) {
  const int rows = a.B * a.H * a.n_q;
  hipLaunchKernelGGL(hybrid_select_reg_kernel<NPAD>, dim3((rows + 3) / 4), dim3(256), 0, st,
                     a.logits, rows, a.n_k, a.words, a.K_k, a.keep_all, a.p, a.bits, a.idx,
                     a.cnt);
  return hipGetLastError();
}

// one row per workgroup. The dynamic-LDS limit of every instantiation (the
// 4096-entry rows need 73 KiB) is raised together, once per device, on the
// first mask call of any width, so that a later call of another width makes
// no attribute change (which could otherwise fall inside a graph capture)
constexpr int kMaxDevices = 64;

template <int NPAD>
hipError_t raise_select_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&hybrid_select_kernel<NPAD>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)select_lds_bytes(NPAD));
}

hipError_t select_lds_ready() {
  static std::once_flag once[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    hipError_t r = raise_select_lds<1024>();
    if (r == hipSuccess) r = raise_select_lds<2048>();
    if (r == hipSuccess) r = raise_select_lds<4096>();
    err[dev] = r;
  });
  return err[dev];
}

template <int NPAD>
hipError_t launch_select(const MaskLaunch& a, hipStream_t st) {
  const int rows = a.B * a.H * a.n_q;
  hipLaunchKernelGGL(hybrid_select_kernel<NPAD>, dim3(rows), dim3(select_threads(NPAD)),
                     select_lds_bytes(NPAD), st, a.logits, rows, a.n_k, a.words, a.K_k,
                     a.keep_all, a.p, a.bits, a.idx, a.cnt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scores_f64(const double* x, const double* y, double* out, int BH, int nx,
                             int ny, int d, double sc, hipStream_t st) {
  const int tq = (nx + 31) / 32, tk = (ny + 31) / 32, tiles = BH * tq * tk;
  if (d == 128)
    hipLaunchKernelGGL(block_logits_kernel<128>, dim3((tiles + 3) / 4), dim3(kThreads), 0, st, x,
                       y, out, nx, ny, tq, tk, tiles, sc);
  else
    hipLaunchKernelGGL(block_logits_kernel<64>, dim3((tiles + 3) / 4), dim3(kThreads), 0, st, x,
                       y, out, nx, ny, tq, tk, tiles, sc);
  return hipGetLastError();
}

constexpr int kRegSelectMinRows = 1024;

hipError_t launch_select_rows(const MaskLaunch& a, hipStream_t st) {
  hipError_t e = select_lds_ready();
  if (e != hipSuccess) return e;
  switch (a.npad) {
    case 64: return launch_select_reg<64>(a, st);
    case 128: return launch_select_reg<128>(a, st);
    case 256: return launch_select_reg<256>(a, st);
    case 512: return launch_select_reg<512>(a, st);
    // 1024 / 2048 entries: one wave per row needs about a thousand rows to
    // fill the chip; with fewer, a workgroup per row (the LDS sort) is faster
    case 1024:
      return a.B * a.H * a.n_q >= kRegSelectMinRows ? launch_select_reg<1024>(a, st)
                                                      : launch_select<1024>(a, st);
    case 2048:
      return a.B * a.H * a.n_q >= kRegSelectMinRows ? launch_select_reg<2048>(a, st)
                                                      : launch_select<2048>(a, st);
    default: return launch_select<4096>(a, st);
  }
}

hipError_t launch_mask(const MaskLaunch& a, hipStream_t st) {
  const int BH = a.B * a.H;
  auto scores = [&](const double* x, const double* y, double* out, int nx, int ny, double sc) {
    const int tq = (nx + 31) / 32, tk = (ny + 31) / 32, tiles = BH * tq * tk;
    if (a.d == 128)
      hipLaunchKernelGGL(block_logits_kernel<128>, dim3((tiles + 3) / 4), dim3(kThreads), 0, st,
                         x, y, out, nx, ny, tq, tk, tiles, sc);
    else
      hipLaunchKernelGGL(block_logits_kernel<64>, dim3((tiles + 3) / 4), dim3(kThreads), 0, st,
                         x, y, out, nx, ny, tq, tk, tiles, sc);
  };
  if (a.phase != 2) {
    const dim3 grid(a.n_q + a.n_k, BH);
    if (a.qc) {
      if (a.d == 128)
        hipLaunchKernelGGL((pool_mean_kernel<128, true>), grid, dim3(kThreads), 0, st, a.q, a.k,
                           a.qbar, a.kbar, a.N, a.block_q, a.block_k, a.n_q, a.n_k, a.qc, a.kc,
                           a.qsc, a.ksc);
      else
        hipLaunchKernelGGL((pool_mean_kernel<64, true>), grid, dim3(kThreads), 0, st, a.q, a.k,
                           a.qbar, a.kbar, a.N, a.block_q, a.block_k, a.n_q, a.n_k, a.qc, a.kc,
                           a.qsc, a.ksc);
    } else if (a.d == 128) {
      hipLaunchKernelGGL((pool_mean_kernel<128>), grid, dim3(kThreads), 0, st, a.q, a.k, a.qbar,
                         a.kbar, a.N, a.block_q, a.block_k, a.n_q, a.n_k, nullptr, nullptr,
                         nullptr, nullptr);
    } else {
      hipLaunchKernelGGL((pool_mean_kernel<64>), grid, dim3(kThreads), 0, st, a.q, a.k, a.qbar,
                         a.kbar, a.N, a.block_q, a.block_k, a.n_q, a.n_k, nullptr, nullptr,
                         nullptr, nullptr);
    }
    if (a.phase == 1) return hipGetLastError();
  }
  const double* qs = a.qbar;
  const double* ks = a.kbar;
  if (a.wq) {  // router: project the pooled rows first (float64, scale 1)
    const dim3 wgrid((a.d * a.d + kThreads - 1) / kThreads, BH);
    hipLaunchKernelGGL(router_weights_kernel, wgrid, dim3(kThreads), 0, st, a.wq, a.wqT, a.H, a.d);
    hipLaunchKernelGGL(router_weights_kernel, wgrid, dim3(kThreads), 0, st, a.wk, a.wkT, a.H, a.d);
    scores(a.qbar, a.wqT, a.qbar_p, a.n_q, a.d, 1.0);
    scores(a.kbar, a.wkT, a.kbar_p, a.n_k, a.d, 1.0);
    qs = a.qbar_p;
    ks = a.kbar_p;
  }
  scores(qs, ks, a.logits, a.n_q, a.n_k, a.scale);
  return launch_select_rows(a, st);
}

}  // namespace sparge

