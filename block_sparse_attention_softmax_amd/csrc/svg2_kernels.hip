// SVG2's semantic-aware sparse attention ("Sparse VideoGen2" page, section 2):
//
//  1. k-means on the query tokens (C_q clusters) and, independently, on the
//     key tokens (C_k clusters): Lloyd's rounds in float64 from centroids at
//     tokens floor(c N / C); distances |c|^2 - 2 x.c on the float64 matrix
//     cores with the argmin (ties to the lower cluster) taken in the same
//     kernel, so no distance matrix is stored; centroids the mean of their
//     members in token order.
//  2. the permutation: a stable counting sort of the tokens by cluster, so
//     each cluster is contiguous (ranks inside 64-token chunks by lane
//     comparisons, per-chunk counts, scans; no atomics, so the order is
//     deterministic).
//  3. centroid Top-p: scale * c_q . c_k plus ln |cluster| (a cluster weighs as
//     many tokens as it holds) and the mask's hybrid selection, Top-k reduced
//     to one cluster.
//  4. attention over variable-size clusters: every cluster is padded to whole
//     tiles (query clusters to block_q rows, key clusters to 64 keys), the
//     permuted Q, K, V are gathered into those padded layouts, each query tile
//     walks the 64-key chunks of its cluster's selected key clusters with the
//     keys past a cluster's end masked, and the output rows are written back
//     to their original positions (the inverse permutation).
#include <algorithm>

#include "internal.h"
#include "tiles.h"

namespace sparge {
namespace {

// x (bf16) -> float64, elementwise.
__global__ __launch_bounds__(256) void to_f64_kernel(const uint16_t* __restrict__ x,
                                                     double* __restrict__ y, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    y[e] = (double)__uint_as_float((uint32_t)x[e] << 16);
}

__global__ __launch_bounds__(256) void fill_i32_zero_kernel(int32_t* __restrict__ p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    p[e] = 0;
}

// sum of v over the D threads of a workgroup (D = 64 or 128)
template <int D>
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = red[0];
  if (D == 128) s += red[1];
  __syncthreads();
  return s;
}

// ------------------------------------------------------------- k-means
// centroid c = token floor(c N / C); |c|^2. Grid (C, B*H), D threads.
template <int D>
__global__ __launch_bounds__(D) void km_init_kernel(const double* __restrict__ x,
                                                    double* __restrict__ cent,
                                                    double* __restrict__ cnorm, int N, int C) {
  __shared__ double red[2];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const size_t tok = (size_t)c * N / C;
  const double v = x[((size_t)bh * N + tok) * D + t];
  cent[((size_t)bh * C + c) * D + t] = v;
  const double s = block_sum<D>(v * v, red);
  if (t == 0) cnorm[(size_t)bh * C + c] = s;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// assign[t] = argmin_c (|c|^2 - 2 x_t . c), ties to the lower c, without
// storing the distances. Workgroup (64 tokens, b, h): wave w holds tokens
// 16 w .. 16 w + 15 in registers (lane: token 16 w + lane % 16, channels
// 8 s + 2 (lane / 16) + 0..1), the centroids stream through LDS 64 at a time
// (rows padded by two doubles so that 16 lanes reading 16 rows hit different
// banks), and each lane keeps the best of its column of every 16 x 16 product
// for the 4 tokens it holds; the 16 lanes of a token group merge at the end.
// The float64 products run in the instruction order of block_logits_kernel
// (two 16x16x4 steps per 8 channels, per accumulator), so every distance has
// the bits of the distance-matrix route it replaces.
template <int D>
__global__ __launch_bounds__(256, 2) void km_assign_kernel(const double* __restrict__ x,
                                                           const double* __restrict__ cent,
                                                           const double* __restrict__ cnorm,
                                                           int32_t* __restrict__ assign, int N,
                                                           int C) {
  constexpr int CT = 64, RP = D + 2;  // centroids per tile; LDS row (doubles)
  __shared__ __align__(16) double cs[CT * RP];
  __shared__ double cn[CT];
  const int bh = blockIdx.y, t0 = blockIdx.x * 64;
  const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
  const int r = lane & 15, g = lane >> 4;
  const size_t xb = (size_t)bh * N;
  const int tok = min(t0 + 16 * wave + r, N - 1);  // tokens past N are computed, not stored
  double2 xr[D / 8];
#pragma unroll
  for (int s = 0; s < D / 8; ++s)
    xr[s] = *reinterpret_cast<const double2*>(x + (xb + tok) * D + 8 * s + 2 * g);
  double best[4] = {INFINITY, INFINITY, INFINITY, INFINITY};
  int bi[4] = {C, C, C, C};
  const double* cb0 = cent + (size_t)bh * C * D;
  for (int cb = 0; cb < C; cb += CT) {
    __syncthreads();  // the previous tile is consumed
    for (int p = th; p < CT * D / 2; p += 256) {
      const int row = p / (D / 2), c2 = p % (D / 2);
      const int cr = min(cb + row, C - 1);
      *reinterpret_cast<double2*>(cs + row * RP + 2 * c2) =
          *reinterpret_cast<const double2*>(cb0 + (size_t)cr * D + 2 * c2);
    }
    if (th < CT) cn[th] = cnorm[(size_t)bh * C + min(cb + th, C - 1)];
    __syncthreads();
    f64x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int s = 0; s < D / 8; ++s) {
      double2 y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        y[b] = *reinterpret_cast<const double2*>(cs + (16 * b + r) * RP + 8 * s + 2 * g);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[s].x, y[b].x, acc[b], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[s].y, y[b].y, acc[b], 0, 0, 0);
    }
    // lane: tokens 4 e + g of the wave's 16, centroid cb + 16 b + r (increasing)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = cb + 16 * b + r;
      if (c < C) {
        const double cnc = cn[16 * b + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double v = cnc - 2.0 * acc[b][e];
          if (v < best[e]) {
            best[e] = v;
            bi[e] = c;
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const double ob = __shfl_xor(best[e], off);
      const int oi = __shfl_xor(bi[e], off);
      if (ob < best[e] || (ob == best[e] && oi < bi[e])) {
        best[e] = ob;
        bi[e] = oi;
      }
    }
    const int t = t0 + 16 * wave + 4 * e + g;
    if (r == 0 && t < N) assign[xb + t] = bi[e];
  }
}

// Stable counting sort by cluster, step 1: per 64-token chunk (one wave),
// each token's rank among the earlier tokens of its cluster in the chunk, and
// the chunk's count of each cluster (written by the cluster's last token;
// counts start at zero).
__global__ __launch_bounds__(256) void km_rank_kernel(const int32_t* __restrict__ assign,
                                                      int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ ccount, int N, int C,
                                                      int nch, size_t total_chunks) {
  const size_t wid = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= total_chunks) return;
  const size_t bh = wid / nch;
  const int ch = (int)(wid % nch), t = ch * 64 + lane;
  const int a = t < N ? assign[bh * N + t] : -1;
  int before = 0, after = 0;
  for (int l = 0; l < 64; ++l) {
    const int o = __shfl(a, l);
    before += (l < lane && o == a) ? 1 : 0;
    after += (l > lane && o == a) ? 1 : 0;
  }
  if (t < N) {
    rank[bh * N + t] = before;
    if (after == 0) ccount[(bh * nch + ch) * C + a] = before + 1;
  }
}

// Step 2: ccount[bh][ch][c] becomes the number of tokens of cluster c in the
// chunks before ch, and size[c] the cluster's total. Workgroup (64 clusters,
// b, h): lanes over clusters (coalesced rows), the 4 waves over quarters of
// the chunks, their sums combined through LDS.
__global__ __launch_bounds__(256) void km_colscan_kernel(int32_t* __restrict__ ccount,
                                                         int32_t* __restrict__ size, int C,
                                                         int nch) {
  __shared__ int part[4][64];
  const int bh = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int q = (nch + 3) / 4, ch0 = min(wave * q, nch), ch1 = min(ch0 + q, nch);
  int32_t* col = ccount + (size_t)bh * nch * C + c;
  int sum = 0;
  if (c < C)
    for (int ch = ch0; ch < ch1; ++ch) sum += col[(size_t)ch * C];
  part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += part[w][lane];
  if (c < C) {
    for (int ch = ch0; ch < ch1; ++ch) {
      const int v = col[(size_t)ch * C];
      col[(size_t)ch * C] = run;
      run += v;
    }
    if (wave == 3) size[(size_t)bh * C + c] = run;
  }
}

// off[bh][c] = the clusters before c in size order, off[bh][C] = N. One
// workgroup per (b, h), 256 clusters per pass with a carry.
__global__ __launch_bounds__(256) void km_offsets_kernel(const int32_t* __restrict__ size,
                                                         int32_t* __restrict__ off, int C) {
  __shared__ int wsum[4];
  const int bh = blockIdx.x, th = threadIdx.x, lane = th & 63, wave = th >> 6;
  int carry = 0;
  for (int base = 0; base < C; base += 256) {
    const int c = base + th;
    const int v = c < C ? size[(size_t)bh * C + c] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    if (c < C) off[(size_t)bh * (C + 1) + c] = carry + wbase + incl - v;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();  // wsum is reused
  }
  if (th == 0) off[(size_t)bh * (C + 1) + C] = carry;
}

// Step 3: perm[off[c] + base[chunk][c] + rank] = token.
__global__ __launch_bounds__(256) void km_scatter_kernel(const int32_t* __restrict__ assign,
                                                         const int32_t* __restrict__ rank,
                                                         const int32_t* __restrict__ ccount,
                                                         const int32_t* __restrict__ off,
                                                         int32_t* __restrict__ perm, int N, int C,
                                                         int nch, size_t total) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const size_t bh = e / N;
  const int t = (int)(e % N), a = assign[e];
  const int pos = off[bh * (C + 1) + a] + ccount[(bh * nch + t / 64) * C + a] + rank[e];
  perm[bh * N + pos] = t;
}

// Centroid c = the mean of its members in token order (float64); an empty
// cluster keeps its centroid; |c|^2. Grid (C, B*H), D threads.
template <int D>
__global__ __launch_bounds__(D) void km_update_kernel(const double* __restrict__ x,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ size,
                                                      const int32_t* __restrict__ off,
                                                      double* __restrict__ cent,
                                                      double* __restrict__ cnorm, int N, int C) {
  __shared__ double red[2];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int n = size[(size_t)bh * C + c], o0 = off[(size_t)bh * (C + 1) + c];
  double* cp = cent + ((size_t)bh * C + c) * D + t;
  double v = *cp;
  if (n > 0) {
    double acc = 0.0;
    for (int m = 0; m < n; ++m) acc += x[((size_t)bh * N + perm[(size_t)bh * N + o0 + m]) * D + t];
    v = acc / n;
    *cp = v;
  }
  const double s = block_sum<D>(v * v, red);
  if (t == 0) cnorm[(size_t)bh * C + c] = s;
}

// ------------------------------------------------------- centroid Top-p
// logits[bh][i][j] += ln size_k[j] (-inf for an empty key cluster).
__global__ __launch_bounds__(256) void svg2_weigh_kernel(double* __restrict__ logits,
                                                         const int32_t* __restrict__ ksize,
                                                         int Cq, int Ck, size_t total) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const size_t bh = e / ((size_t)Cq * Ck);
  const int j = (int)(e % Ck);
  const int n = ksize[bh * Ck + j];
  logits[e] = n > 0 ? logits[e] + log((double)n) : -INFINITY;
}

// ------------------------------------------------------------- layouts
// Per (b, h): padded offsets of the query clusters (whole tiles of BQ rows)
// and key clusters (whole 64-key chunks), the cluster of every query tile,
// the valid keys of every chunk, and the tile count.
__global__ __launch_bounds__(64) void svg2_layout_kernel(
    const int32_t* __restrict__ qsize, const int32_t* __restrict__ ksize,
    int32_t* __restrict__ qpad_off, int32_t* __restrict__ kpad_off,
    int32_t* __restrict__ tile_cluster, int32_t* __restrict__ chunk_valid,
    int32_t* __restrict__ n_tiles, int Cq, int Ck, int BQ, int max_tiles, int max_chunks) {
  const int bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  int tiles = 0;
  for (int c = 0; c < Cq; ++c) {
    qpad_off[(size_t)bh * Cq + c] = tiles * BQ;
    const int nt = (qsize[(size_t)bh * Cq + c] + BQ - 1) / BQ;
    for (int u = 0; u < nt; ++u) tile_cluster[(size_t)bh * max_tiles + tiles + u] = c;
    tiles += nt;
  }
  n_tiles[bh] = tiles;
  int chunks = 0;
  for (int c = 0; c < Ck; ++c) {
    const int n = ksize[(size_t)bh * Ck + c], nc = (n + BK - 1) / BK;
    kpad_off[(size_t)bh * Ck + c] = chunks * BK;
    for (int u = 0; u < nc; ++u)
      chunk_valid[(size_t)bh * max_chunks + chunks + u] = min(BK, n - u * BK);
    chunks += nc;
  }
}

// Per (b, h, query cluster), one wave: the chunks of its selected key
// clusters, in the selection's order.
__global__ __launch_bounds__(256) void svg2_lists_kernel(const int32_t* __restrict__ sidx,
                                                         const int32_t* __restrict__ scnt,
                                                         const int32_t* __restrict__ kpad_off,
                                                         const int32_t* __restrict__ ksize,
                                                         int32_t* __restrict__ lists,
                                                         int32_t* __restrict__ list_cnt, int Cq,
                                                         int Ck, int max_chunks, size_t rows) {
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const size_t bh = row / Cq;
  const int cnt = scnt[row];
  int pos = 0;
  for (int e = 0; e < cnt; ++e) {
    const int j = sidx[row * Ck + e];
    const int nc = (ksize[bh * Ck + j] + BK - 1) / BK, base = kpad_off[bh * Ck + j] / BK;
    for (int u = lane; u < nc; u += 64) lists[row * max_chunks + pos + u] = base + u;
    pos += nc;
  }
  if (lane == 0) list_cnt[row] = pos;
}

// Gather the rows of each cluster (in permuted order) into its padded slot;
// padding rows are zero. Grid (clusters, B*H), 256 threads, 16-byte copies.
template <int D>
__global__ __launch_bounds__(256) void svg2_gather_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ off,
                                                          const int32_t* __restrict__ size,
                                                          const int32_t* __restrict__ pad_off,
                                                          uint16_t* __restrict__ xp, int N,
                                                          int C, int pad, int NP) {
  constexpr int CPR = D / 8;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int n = size[(size_t)bh * C + c], np = (n + pad - 1) / pad * pad;
  const int o0 = off[(size_t)bh * (C + 1) + c], p0 = pad_off[(size_t)bh * C + c];
  for (int e = threadIdx.x; e < np * CPR; e += 256) {
    const int r = e / CPR, ch = e % CPR;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r < n) {
      const int tok = perm[(size_t)bh * N + o0 + r];
      u = *reinterpret_cast<const uint4*>(x + ((size_t)bh * N + tok) * D + ch * 8);
    }
    *reinterpret_cast<uint4*>(xp + ((size_t)bh * NP + p0 + r) * D + ch * 8) = u;
  }
}

// ------------------------------------------------------------ attention
// One workgroup per padded query tile (BQ rows of one cluster), BQ/32 waves of
// 32 queries: S^T = K Q^T and O^T += V^T P^T on bf16 MFMA as in the sparse
// kernel, online softmax with an exact running maximum, K rows and packed V^T
// of each 64-key chunk double-buffered by direct-to-LDS copies; keys past the
// chunk's valid count get -inf; rows go back to their tokens.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 2) void svg2_attn_kernel(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vtp, const int32_t* __restrict__ chunk_valid,
    const int32_t* __restrict__ tile_cluster, const int32_t* __restrict__ n_tiles,
    const int32_t* __restrict__ lists, const int32_t* __restrict__ list_cnt,
    const int32_t* __restrict__ perm_q, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ size_q, const int32_t* __restrict__ qpad_off,
    uint16_t* __restrict__ o, int N, int NQP, int NKP, int Cq, int max_tiles, int max_chunks,
    float c) {
  using T = Tile<D>;
  constexpr int NT = BQ * 2, DT = D / 32, KSTEPS = D / 16;
  constexpr int KU = 64 * T::KCPR / NT, VU = D * T::VCPR / NT;
  __shared__ __align__(16) unsigned char smem[4 * T::BYTES];
  const int bh = blockIdx.x / max_tiles, tile = blockIdx.x % max_tiles;
  if (tile >= n_tiles[bh]) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int cq = tile_cluster[(size_t)bh * max_tiles + tile];
  const int prow = tile * BQ + wave * 32 + l32;  // row of the padded permuted Q
  const int local = prow - qpad_off[(size_t)bh * Cq + cq];
  const bool valid = local < size_q[(size_t)bh * Cq + cq];

  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qr = qp + ((size_t)bh * NQP + prow) * D + 8 * h2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
  }
  const size_t lrow = (size_t)bh * Cq + cq;
  const int count = list_cnt[lrow];
  const int32_t* ids = lists + lrow * max_chunks;

  uint32_t kofs[KU], vofs[VU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int p = u * NT + threadIdx.x, r = p / T::KCPR;
    kofs[u] = (uint32_t)(r * D + T::kchunk(r, p % T::KCPR) * 8);
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = u * NT + threadIdx.x, r = p / T::VCPR;
    vofs[u] = (uint32_t)(r * BK + T::vchunk(r, p % T::VCPR) * 8);
  }
  auto issue = [&](int j, int b) {
    const uint16_t* ks = kp + ((size_t)bh * NKP + (size_t)j * BK) * D;
    const uint16_t* vs = vtp + ((size_t)bh * (NKP / BK) + j) * (size_t)D * BK;
#pragma unroll
    for (int u = 0; u < KU; ++u) dma16(ks + kofs[u], smem + b * T::BYTES + (u * NT + wave * 64) * 16);
#pragma unroll
    for (int u = 0; u < VU; ++u)
      dma16(vs + vofs[u], smem + (2 + b) * T::BYTES + (u * NT + wave * 64) * 16);
  };

  floatx16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;
  if (count > 0) issue(ids[0], 0);
  for (int e = 0; e < count; ++e) {
    const int j = ids[e];
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of chunk e landed
    __syncthreads();                     // all copies landed; the other buffers are free
    if (e + 1 < count) issue(ids[e + 1], (e + 1) & 1);
    const unsigned char* kt = smem + (e & 1) * T::BYTES;
    const unsigned char* vt = smem + (2 + (e & 1)) * T::BYTES;
    floatx16 S[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[tau][r] = 0.0f;
      const int kr = 32 * tau + l32;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 a = lds_read16(kt + kr * T::KROWB + T::kchunk(kr, 2 * s + h2) * 16);
        S[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], S[tau], 0, 0, 0);
      }
    }
    const int nvalid = chunk_valid[(size_t)bh * max_chunks + j];
    float mloc = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * tau + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (key >= nvalid) S[tau][r] = -INFINITY;
        mloc = fmaxf(mloc, S[tau][r]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m, mloc);
    if (__any(m_new > m)) {
      const float f = m_new > m ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.0f;
      lsum *= f;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= f;
      m = m_new;
    }
    const float mc = m * c;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[tau][r] = __builtin_amdgcn_exp2f(fmaf(S[tau][r], c, -mc));
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        const bf16x8 pb = pack_bf16x8(S[tau], 8 * hk);
        lsum = row_sum_bf16x8(pb, lsum);
        const int ch = 4 * tau + 2 * hk + h2;
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int row = 32 * i + l32;
          const bf16x8 a = lds_read16(vt + row * T::VROWB + T::vchunk(row, ch) * 16);
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[i], 0, 0, 0);
        }
      }
  }
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (valid) {
    const int tok = perm_q[(size_t)bh * N + off_q[(size_t)bh * (Cq + 1) + cq] + local];
    uint16_t* orow = o + ((size_t)bh * N + tok) * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * i + 8 * g + 4 * h2;
        uint2 pk;
        pk.x = pack2_bf16(oacc[i][4 * g + 0] * inv, oacc[i][4 * g + 1] * inv);
        pk.y = pack2_bf16(oacc[i][4 * g + 2] * inv, oacc[i][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
  }
}

// --------------------------------------------------------------- driver
template <int D>
hipError_t kmeans_run(const Svg2Launch& a, const double* x, int C, double* cent, double* cnorm,
                      int32_t* assign, int32_t* size, int32_t* off, int32_t* perm, hipStream_t s) {
  const int BH = a.B * a.H, nch = (a.N + 63) / 64;
  const size_t rows = (size_t)BH * a.N, chunks = (size_t)BH * nch, cc = chunks * C;
  hipLaunchKernelGGL((km_init_kernel<D>), dim3(C, BH), dim3(D), 0, s, x, cent, cnorm, a.N, C);
  for (int it = 0; it <= a.iters; ++it) {
    hipLaunchKernelGGL((km_assign_kernel<D>), dim3(nch, BH), dim3(256), 0, s, x, cent, cnorm,
                       assign, a.N, C);
    hipLaunchKernelGGL(fill_i32_zero_kernel, dim3((unsigned)std::min<size_t>((cc + 255) / 256, 4096)),
                       dim3(256), 0, s, a.ccount, cc);
    hipLaunchKernelGGL(km_rank_kernel, dim3((unsigned)((chunks + 3) / 4)), dim3(256), 0, s, assign,
                       a.rank, a.ccount, a.N, C, nch, chunks);
    hipLaunchKernelGGL(km_colscan_kernel, dim3((C + 63) / 64, BH), dim3(256), 0, s, a.ccount, size,
                       C, nch);
    hipLaunchKernelGGL(km_offsets_kernel, dim3(BH), dim3(256), 0, s, size, off, C);
    hipLaunchKernelGGL(km_scatter_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                       assign, a.rank, a.ccount, off, perm, a.N, C, nch, rows);
    if (it < a.iters)
      hipLaunchKernelGGL((km_update_kernel<D>), dim3(C, BH), dim3(D), 0, s, x, perm, size, off,
                         cent, cnorm, a.N, C);
  }
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_svg2_t(const Svg2Launch& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const size_t n = (size_t)BH * a.N * D;
  hipLaunchKernelGGL(to_f64_kernel, dim3(4096), dim3(256), 0, s, a.q, a.xq, n);
  hipLaunchKernelGGL(to_f64_kernel, dim3(4096), dim3(256), 0, s, a.k, a.xk, n);
  hipError_t e = kmeans_run<D>(a, a.xq, a.Cq, a.centq, a.normq, a.assign_q, a.size_q, a.off_q,
                               a.perm_q, s);
  if (e == hipSuccess)
    e = kmeans_run<D>(a, a.xk, a.Ck, a.centk, a.normk, a.assign_k, a.size_k, a.off_k, a.perm_k, s);
  if (e != hipSuccess) return e;
  // centroid Top-p
  e = launch_scores_f64(a.centq, a.centk, a.clog, BH, a.Cq, a.Ck, D, (double)a.scale, s);
  if (e != hipSuccess) return e;
  const size_t nl = (size_t)BH * a.Cq * a.Ck;
  hipLaunchKernelGGL(svg2_weigh_kernel, dim3((unsigned)((nl + 255) / 256)), dim3(256), 0, s, a.clog,
                     a.size_k, a.Cq, a.Ck, nl);
  MaskLaunch m{};
  m.B = a.B; m.H = a.H; m.n_q = a.Cq; m.n_k = a.Ck;
  int npad = 64;
  while (npad < a.Ck) npad *= 2;
  m.npad = npad;
  m.words = (a.Ck + 31) / 32;
  m.K_k = 1;
  m.keep_all = a.p >= 1.0 ? 1 : 0;
  m.p = a.p;
  m.logits = a.clog;
  m.bits = a.sbits;
  m.idx = a.sidx;
  m.cnt = a.scnt;
  e = launch_select_rows(m, s);
  if (e != hipSuccess) return e;
  // padded layouts, chunk lists, gathers
  hipLaunchKernelGGL(svg2_layout_kernel, dim3(BH), dim3(64), 0, s, a.size_q, a.size_k,
                     a.qpad_off, a.kpad_off, a.tile_cluster, a.chunk_valid, a.n_tiles, a.Cq, a.Ck,
                     BQ, a.max_tiles, a.max_chunks);
  const size_t lrows = (size_t)BH * a.Cq;
  hipLaunchKernelGGL(svg2_lists_kernel, dim3((unsigned)((lrows + 3) / 4)), dim3(256), 0, s, a.sidx,
                     a.scnt, a.kpad_off, a.size_k, a.lists, a.list_cnt, a.Cq, a.Ck, a.max_chunks,
                     lrows);
  const int NQP = a.max_tiles * BQ, NKP = a.max_chunks * BK;
  hipLaunchKernelGGL((svg2_gather_kernel<D>), dim3(a.Cq, BH), dim3(256), 0, s, a.q, a.perm_q,
                     a.off_q, a.size_q, a.qpad_off, a.qp, a.N, a.Cq, BQ, NQP);
  hipLaunchKernelGGL((svg2_gather_kernel<D>), dim3(a.Ck, BH), dim3(256), 0, s, a.k, a.perm_k,
                     a.off_k, a.size_k, a.kpad_off, a.kp, a.N, a.Ck, BK, NKP);
  hipLaunchKernelGGL((svg2_gather_kernel<D>), dim3(a.Ck, BH), dim3(256), 0, s, a.v, a.perm_k,
                     a.off_k, a.size_k, a.kpad_off, a.vp, a.N, a.Ck, BK, NKP);
  hipLaunchKernelGGL((pack_kernel<D, false>), dim3(a.max_chunks, BH), dim3(2 * D), 0, s, a.vp,
                     nullptr, a.vtp, nullptr, NKP, a.max_chunks, nullptr, a.H);
  hipLaunchKernelGGL((svg2_attn_kernel<D, BQ>), dim3(BH * a.max_tiles), dim3(BQ * 2), 0, s, a.qp,
                     a.kp, a.vtp, a.chunk_valid, a.tile_cluster, a.n_tiles, a.lists, a.list_cnt,
                     a.perm_q, a.off_q, a.size_q, a.qpad_off, a.o, a.N, NQP, NKP, a.Cq,
                     a.max_tiles, a.max_chunks, a.scale * 1.4426950408889634f);
  return hipGetLastError();
}

}  // namespace

size_t svg2_workspace_bytes(int B, int H, int N, int d, int block_q, int Cq, int Ck) {
  Svg2Launch a{};
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q; a.Cq = Cq; a.Ck = Ck;
  return svg2_layout(a, nullptr);
}

size_t svg2_layout(Svg2Launch& a, unsigned char* w) {
  const size_t BH = (size_t)a.B * a.H, N = a.N, d = a.d, nch = (N + 63) / 64;
  const size_t Cm = (size_t)std::max(a.Cq, a.Ck);
  a.max_tiles = (int)((N + a.block_q - 1) / a.block_q + a.Cq);
  a.max_chunks = (int)(nch + a.Ck);
  const size_t NQP = (size_t)a.max_tiles * a.block_q, NKP = (size_t)a.max_chunks * BK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = w ? w + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  a.xq = reinterpret_cast<double*>(take(BH * N * d * 8));
  a.xk = reinterpret_cast<double*>(take(BH * N * d * 8));
  a.centq = reinterpret_cast<double*>(take(BH * a.Cq * d * 8));
  a.centk = reinterpret_cast<double*>(take(BH * a.Ck * d * 8));
  a.normq = reinterpret_cast<double*>(take(BH * a.Cq * 8));
  a.normk = reinterpret_cast<double*>(take(BH * a.Ck * 8));
  a.assign_q = reinterpret_cast<int32_t*>(take(BH * N * 4));
  a.assign_k = reinterpret_cast<int32_t*>(take(BH * N * 4));
  a.rank = reinterpret_cast<int32_t*>(take(BH * N * 4));
  a.ccount = reinterpret_cast<int32_t*>(take(BH * nch * Cm * 4));
  a.size_q = reinterpret_cast<int32_t*>(take(BH * a.Cq * 4));
  a.size_k = reinterpret_cast<int32_t*>(take(BH * a.Ck * 4));
  a.off_q = reinterpret_cast<int32_t*>(take(BH * (a.Cq + 1) * 4));
  a.off_k = reinterpret_cast<int32_t*>(take(BH * (a.Ck + 1) * 4));
  a.perm_q = reinterpret_cast<int32_t*>(take(BH * N * 4));
  a.perm_k = reinterpret_cast<int32_t*>(take(BH * N * 4));
  a.clog = reinterpret_cast<double*>(take(BH * a.Cq * a.Ck * 8));
  a.sbits = reinterpret_cast<uint32_t*>(take(BH * a.Cq * ((a.Ck + 31) / 32) * 4));
  a.sidx = reinterpret_cast<int32_t*>(take(BH * a.Cq * a.Ck * 4));
  a.scnt = reinterpret_cast<int32_t*>(take(BH * a.Cq * 4));
  a.qpad_off = reinterpret_cast<int32_t*>(take(BH * a.Cq * 4));
  a.kpad_off = reinterpret_cast<int32_t*>(take(BH * a.Ck * 4));
  a.tile_cluster = reinterpret_cast<int32_t*>(take(BH * a.max_tiles * 4));
  a.chunk_valid = reinterpret_cast<int32_t*>(take(BH * a.max_chunks * 4));
  a.n_tiles = reinterpret_cast<int32_t*>(take(BH * 4));
  a.lists = reinterpret_cast<int32_t*>(take(BH * a.Cq * a.max_chunks * 4));
  a.list_cnt = reinterpret_cast<int32_t*>(take(BH * a.Cq * 4));
  a.qp = reinterpret_cast<uint16_t*>(take(BH * NQP * d * 2));
  a.kp = reinterpret_cast<uint16_t*>(take(BH * NKP * d * 2));
  a.vp = reinterpret_cast<uint16_t*>(take(BH * NKP * d * 2));
  a.vtp = reinterpret_cast<uint16_t*>(take(BH * NKP * d * 2));
  return off;
}

hipError_t launch_svg2(const Svg2Launch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_svg2_t<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_svg2_t<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_svg2_t<64, 128>(a, s);
  return launch_svg2_t<64, 64>(a, s);
}

}  // namespace sparge
