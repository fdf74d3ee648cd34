// Block mask of the hybrid Top-k + Top-p rule, three kernels:
//
//   pool_mean_kernel    Qbar, Kbar = means of the valid rows of every block
//                       (pooled queries and keys as on the SLA2 page,
//                       section 2B; mean pooling of blocks as the Sparse
//                       VideoGen2 page, section 1, names it). HBM-bound: it
//                       reads Q and K once.
//   block_logits_kernel s = scale * Qbar Kbar^T per head, float64, LDS-tiled.
//   hybrid_select_kernel one workgroup per query-block row: softmax of s,
//                       bitonic sort of (score desc, index asc) in LDS,
//                       float64 prefix sum for Top-p, union with Top-k
//                       (SpargeAttention2 page, sections 1 and 2A), then the
//                       bitmask and the ascending index list.
//
// Everything that decides the mask is float64, so the selection is the one a
// float64 evaluation of the definition gives, up to summation order.
#include "internal.h"

namespace sparge {
namespace {

constexpr int kThreads = 256;

// ----------------------------------------------------------------- pooling
// grid (nblk, B*H); one workgroup per block of `block` rows.
template <int D>
__global__ __launch_bounds__(kThreads) void pool_mean_kernel(
    const uint16_t* __restrict__ x, double* __restrict__ out, int N, int block,
    int nblk) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int RSTEP = kThreads / CH;   // rows handled per pass
  __shared__ double red[kThreads][9];    // +1 pad against bank conflicts

  const int bh = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
  const int c = t % CH, r0 = t / CH;
  const int start = blk * block;
  const int rows = min(block, N - start);
  const uint4* src =
      reinterpret_cast<const uint4*>(x + ((size_t)bh * N + start) * D) + c;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = r0; r < rows; r += RSTEP) {
    const uint4 w = src[(size_t)r * CH];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_lo(ws[e]);
      acc[2 * e + 1] += (double)bf16_hi(ws[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[t][e] = acc[e];
  __syncthreads();
  if (t < D) {
    const int cc = t / 8, e = t % 8;
    double s = 0.0;
    for (int r = 0; r < RSTEP; ++r) s += red[r * CH + cc][e];
    out[((size_t)bh * nblk + blk) * D + t] = s / (double)rows;
  }
}

// ------------------------------------------------------------ block scores
// s[bh][i][j] = scale * sum_c qbar[bh][i][c] * kbar[bh][j][c]
// grid (ceil(n_k/64), ceil(n_q/32), B*H); 256 threads, 2x4 outputs each.
constexpr int LQ = 32, LK = 64, LC = 16;
template <int D>
__global__ __launch_bounds__(kThreads) void block_logits_kernel(
    const double* __restrict__ qbar, const double* __restrict__ kbar,
    double* __restrict__ s, int n_q, int n_k, double scale) {
  __shared__ double qs[LQ][LC + 1];
  __shared__ double ks[LK][LC + 1];
  const int bh = blockIdx.z, i0 = blockIdx.y * LQ, j0 = blockIdx.x * LK;
  const int t = threadIdx.x, ty = t / 16, tx = t % 16;
  const double* qh = qbar + (size_t)bh * n_q * D;
  const double* kh = kbar + (size_t)bh * n_k * D;
  double acc[2][4] = {};
  for (int c0 = 0; c0 < D; c0 += LC) {
    for (int u = t; u < LQ * LC; u += kThreads) {
      const int r = u / LC, cc = u % LC;
      qs[r][cc] = (i0 + r < n_q) ? qh[(size_t)(i0 + r) * D + c0 + cc] : 0.0;
    }
    for (int u = t; u < LK * LC; u += kThreads) {
      const int r = u / LC, cc = u % LC;
      ks[r][cc] = (j0 + r < n_k) ? kh[(size_t)(j0 + r) * D + c0 + cc] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < LC; ++cc) {
      const double a0 = qs[2 * ty][cc], a1 = qs[2 * ty + 1][cc];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double b = ks[tx + 16 * u][cc];
        acc[0][u] = fma(a0, b, acc[0][u]);
        acc[1][u] = fma(a1, b, acc[1][u]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int i = i0 + 2 * ty + rr;
    if (i >= n_q) continue;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + tx + 16 * u;
      if (j < n_k) s[((size_t)bh * n_q + i) * n_k + j] = scale * acc[rr][u];
    }
  }
}

// ------------------------------------------------- workgroup scan helpers
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
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

// Exclusive scan of one value per thread over the 256-thread workgroup.
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* wtot) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const T incl = wave_incl_scan(v, lane);
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  T base = 0;
  for (int u = 0; u < w; ++u) base += wtot[u];
  __syncthreads();
  return base + incl - v;
}

// ----------------------------------------------------------- selection
// One workgroup per query-block row. Dynamic LDS: sv[npad] doubles,
// si[npad] ints, bits[words] uint32.
__global__ __launch_bounds__(kThreads) void hybrid_select_kernel(
    const double* __restrict__ s, int n_k, int npad, int words, int K_k,
    int keep_all, double p, uint32_t* __restrict__ bits_out,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* sv = reinterpret_cast<double*>(smem);
  int* si = reinterpret_cast<int*>(sv + npad);
  uint32_t* wb = reinterpret_cast<uint32_t*>(si + npad);
  __shared__ double dred[4];
  __shared__ int ired[4];
  __shared__ int first_hit;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const size_t row = blockIdx.x;
  const double* srow = s + row * (size_t)n_k;

  // 1. load scores, padding with -inf past n_k; row maximum
  double mx = -INFINITY;
  for (int j = t; j < npad; j += kThreads) {
    const double v = j < n_k ? srow[j] : -INFINITY;
    sv[j] = v;
    si[j] = j;
    mx = fmax(mx, v);
  }
  if (t < words) wb[t] = 0u;
  if (t == 0) first_hit = INT32_MAX;
  mx = wave_max(mx);
  if (lane == 0) dred[w] = mx;
  __syncthreads();
  mx = fmax(fmax(dred[0], dred[1]), fmax(dred[2], dred[3]));
  __syncthreads();

  // 2. softmax normaliser
  double tot = 0.0;
  for (int j = t; j < n_k; j += kThreads) tot += exp(sv[j] - mx);
  tot = wave_sum(tot);
  if (lane == 0) dred[w] = tot;
  __syncthreads();
  tot = (dred[0] + dred[1]) + (dred[2] + dred[3]);

  // 3. bitonic sort: position 0 = highest score, equal scores lower index
  //    first. All (score, index) pairs are distinct, so the order is total.
  for (int kk = 2; kk <= npad; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int pi = t; pi < (npad >> 1); pi += kThreads) {
        const int i = 2 * pi - (pi & (jj - 1));
        const int l = i + jj;
        const double a = sv[i], b = sv[l];
        const int ia = si[i], ib = si[l];
        const bool l_first = (b > a) || (b == a && ib < ia);
        const bool up = (i & kk) == 0;
        if (l_first == up) {
          sv[i] = b; sv[l] = a;
          si[i] = ib; si[l] = ia;
        }
      }
      __syncthreads();
    }
  }

  // 4. Top-p: cumulative probability in sorted order; first prefix >= p
  int m_p = n_k;
  if (!keep_all) {
    if (p <= 0.0) {
      m_p = 0;
    } else {
      const int per = npad / kThreads > 0 ? npad / kThreads : 1;
      const int r0 = t * per;
      double local = 0.0;
      for (int r = r0; r < r0 + per && r < n_k; ++r) local += exp(sv[r] - mx) / tot;
      double base = block_excl_scan(local, dred);
      for (int r = r0; r < r0 + per && r < n_k; ++r) {
        base += exp(sv[r] - mx) / tot;
        if (base >= p) { atomicMin(&first_hit, r + 1); break; }
      }
      __syncthreads();
      if (first_hit != INT32_MAX) m_p = first_hit;
    }
  }
  const int count = max(K_k, m_p);

  // 5. union = first `count` of the order -> bitmask
  for (int r = t; r < count; r += kThreads) {
    const int j = si[r];
    if (j < n_k) atomicOr(&wb[j >> 5], 1u << (j & 31));  // (only non-finite scores reach j >= n_k)
  }
  __syncthreads();

  // 6. emit bitmask, ascending index list and count
  uint32_t word = t < words ? wb[t] : 0u;
  if (t < words) bits_out[row * words + t] = word;
  const int off = block_excl_scan((int)__popc(word), ired);
  int32_t* irow = idx_out + row * (size_t)n_k;
  int pos = off;
  while (word) {
    const int b = __ffs(word) - 1;
    irow[pos++] = t * 32 + b;
    word &= word - 1;
  }
  if (t == 0) cnt_out[row] = count;
}

}  // namespace

hipError_t launch_mask(const MaskLaunch& a, hipStream_t st) {
  const int BH = a.B * a.H;
  if (a.d == 128) {
    hipLaunchKernelGGL(pool_mean_kernel<128>, dim3(a.n_q, BH), dim3(kThreads), 0, st,
                       a.q, a.qbar, a.N, a.block_q, a.n_q);
    hipLaunchKernelGGL(pool_mean_kernel<128>, dim3(a.n_k, BH), dim3(kThreads), 0, st,
                       a.k, a.kbar, a.N, a.block_k, a.n_k);
    hipLaunchKernelGGL(block_logits_kernel<128>,
                       dim3((a.n_k + LK - 1) / LK, (a.n_q + LQ - 1) / LQ, BH),
                       dim3(kThreads), 0, st, a.qbar, a.kbar, a.logits, a.n_q, a.n_k,
                       a.scale);
  } else {
    hipLaunchKernelGGL(pool_mean_kernel<64>, dim3(a.n_q, BH), dim3(kThreads), 0, st,
                       a.q, a.qbar, a.N, a.block_q, a.n_q);
    hipLaunchKernelGGL(pool_mean_kernel<64>, dim3(a.n_k, BH), dim3(kThreads), 0, st,
                       a.k, a.kbar, a.N, a.block_k, a.n_k);
    hipLaunchKernelGGL(block_logits_kernel<64>,
                       dim3((a.n_k + LK - 1) / LK, (a.n_q + LQ - 1) / LQ, BH),
                       dim3(kThreads), 0, st, a.qbar, a.kbar, a.logits, a.n_q, a.n_k,
                       a.scale);
  }
  const size_t lds = (size_t)a.npad * (sizeof(double) + sizeof(int)) +
                     (size_t)a.words * sizeof(uint32_t);
  hipLaunchKernelGGL(hybrid_select_kernel, dim3(BH * a.n_q), dim3(kThreads), lds, st,
                     a.logits, a.n_k, a.npad, a.words, a.K_k, a.keep_all, a.p, a.bits,
                     a.idx, a.cnt);
  return hipGetLastError();
}

}  // namespace sparge
