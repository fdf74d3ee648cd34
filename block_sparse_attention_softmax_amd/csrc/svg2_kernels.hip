// SVG2's semantic-aware sparse attention ("Sparse VideoGen2" page, section 2):
//
//  1. k-means on the query tokens (C_q clusters) and, independently, on the
//     key tokens (C_k clusters): Lloyd's rounds in float64 from centroids at
//     tokens floor(c N / C); the argmin of the float64 distances
//     |c|^2 - 2 x.c (ties to the lower cluster) found by a bf16 matrix-core
//     filter with a proven error bound, the close calls decided by float64
//     matrix-core products, no distance matrix stored; centroids the mean of
//     their members in token order.
//  2. the permutation: a stable counting sort of the tokens by cluster, so
//     each cluster is contiguous (ranks inside 64-token chunks by lane
//     comparisons, per-chunk counts, scans; no atomics, so the order is
//     deterministic).
//  3. centroid Top-p: scale * c_q . c_k plus ln |cluster| (a cluster weighs as
//     many tokens as it holds) and the mask's hybrid selection, Top-k reduced
//     to one cluster.
//  4. attention over variable-size clusters: query clusters are padded to
//     whole tiles of block_q rows, key clusters only to whole 16-key groups;
//     the permuted Q, K, V are gathered into those layouts, each query tile
//     walks 64-key chunks made of four groups of its cluster's selected key
//     clusters (gathered into LDS group by group), with the keys past a
//     group's valid count masked and waves past the cluster's end idle, and
//     the output rows are written back to their original positions (the
//     inverse permutation).
#include <algorithm>
#include <type_traits>

#include "internal.h"
#include "tiles.h"

namespace sparge {
namespace {

// bf16 bits -> float64 (exact)
__device__ __forceinline__ double bf16_f64(uint16_t u) {
  return (double)__uint_as_float((uint32_t)u << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
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
// The tokens are read as bf16 and widened exactly, so every float64 value is
// the token's own. centroid c = token floor(c N / C); |c|^2. Grid (C, B*H),
// D threads.
template <int D>
__global__ __launch_bounds__(D) void km_init_kernel(const uint16_t* __restrict__ x,
                                                    double* __restrict__ cent,
                                                    double* __restrict__ cnorm, int N, int C) {
  __shared__ double red[2];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const size_t tok = (size_t)c * N / C;
  const double v = bf16_f64(x[((size_t)bh * N + tok) * D + t]);
  cent[((size_t)bh * C + c) * D + t] = v;
  const double s = block_sum<D>(v * v, red);
  if (t == 0) cnorm[(size_t)bh * C + c] = s;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// The assignment assign[t] = argmin_c (|c|^2 - 2 x_t . c) over float64
// distances, ties to the lower c, in two passes that give exactly the
// float64 result:
//  (a) km_filter_kernel: every distance on the bf16 matrix cores from the
//      centroid split into two bf16 planes (c = hi + lo + r, |r| <= 2^-16 |c|
//      per channel; x is bf16 already), accumulated in float32. Its error
//      against the float64 distance is bounded by E = 1.25e-4 |x| cmax +
//      2.5e-7 cmax^2 (cmax = the largest |c| of the head): the split residual
//      (2^-16), float32 accumulation of 2 D exact products (at most 2 D
//      roundings of 2^-23 each), and the float32 roundings of |c|^2 and of
//      the difference, with about 30% to spare. A token whose best and
//      second-best approximate distances are more than 2E apart has that
//      best cluster as its unique float64 argmin, and it is written; any
//      other token (and any non-finite or huge value) is listed.
//  (b) km_exact_kernel: the listed tokens only, with the float64 products
//      below, so a close call is decided by the float64 distances.

// Per round: the centroid planes, |c|^2 in float32 (rows padded to whole
// 64-centroid tiles with +inf) and cmax per (b, h) (as float bits, maxed into
// a zeroed word). Workgroup (16 clusters, b, h), 256
// threads: the planes element by element, the 16 norms and their maximum in
// the workgroup, one atomic per workgroup.
constexpr int kPlaneClusters = 16;

template <int D>
__global__ __launch_bounds__(256) void km_planes_kernel(const double* __restrict__ cent,
                                                        const double* __restrict__ cnorm,
                                                        uint16_t* __restrict__ chi,
                                                        uint16_t* __restrict__ clo,
                                                        float* __restrict__ cnf,
                                                        uint32_t* __restrict__ cmax_bits, int C) {
  const int bh = blockIdx.y, c0 = blockIdx.x * kPlaneClusters, t = threadIdx.x;
  const int nc = min(kPlaneClusters, C - c0);
  const size_t base = ((size_t)bh * C + c0) * D;
  for (int e = t; e < nc * D; e += 256) {
    const double v = cent[base + e];
    const uint16_t hi = bf16_rne((float)v);
    chi[base + e] = hi;
    clo[base + e] = bf16_rne((float)(v - bf16_f64(hi)));
  }
  const int cpad = (C + BK - 1) / BK * BK;  // cnf rows per (b, h): whole 64-centroid tiles
  if (c0 + kPlaneClusters >= C)  // the last workgroup of the head: +inf past C
    for (int e = C + t; e < cpad; e += 256) cnf[(size_t)bh * cpad + e] = INFINITY;
  if (t < 64) {
    float nrm = 0.0f;
    if (t < nc) {
      const double cn = cnorm[(size_t)bh * C + c0 + t];
      cnf[(size_t)bh * cpad + c0 + t] = (float)cn;
      nrm = (float)sqrt(cn) * (1.0f + 1e-6f);  // an upper bound of |c|
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nrm = fmaxf(nrm, __shfl_xor(nrm, off));
    if (t == 0) atomicMax(&cmax_bits[bh], __float_as_uint(nrm));
  }
}

// (a) Workgroup (256 tokens, b, h), 4 waves of 64 tokens (two 32-token
// halves). S^T = C_tile X^T as in the attention's S^T = K Q^T: the token
// fragments stay in registers (one token per lane column and half), the
// planes of 64 centroids at a time are copied global -> LDS (swizzled K-tile
// layout, double-buffered, rows past C repeat row C - 1 and are skipped), each
// plane fragment read from LDS feeds both halves, and the next k-step's
// fragments are read while the current one multiplies. Each lane keeps the
// best, its cluster and the second best of its 16-row slices per half; the
// two half-waves merge at the end.
template <int D>
__global__ __launch_bounds__(256, 2) void km_filter_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ chi,
    const uint16_t* __restrict__ clo, const float* __restrict__ cnf,
    const uint32_t* __restrict__ cmax_bits, int32_t* __restrict__ assign,
    int32_t* __restrict__ flag_list, int32_t* __restrict__ flag_cnt, int N, int C) {
  using T = Tile<D>;
  constexpr int NW = 4, KSTEPS = D / 16;
  constexpr int LOADS = BK * D / 8 / 64 / NW;  // 16-byte copies per wave and plane tile
  // [buffer][plane] tiles, then |c|^2 of the two buffers' centroids
  __shared__ __align__(16) unsigned char smem[4 * T::BYTES + 2 * BK * 4];
  unsigned char* const cns = smem + 4 * T::BYTES;
  const int bh = blockIdx.y, t0 = blockIdx.x * 256;
  const int th = threadIdx.x, lane = th & 63;
  const int wave = __builtin_amdgcn_readfirstlane(th >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t xb = (size_t)bh * N;
  bf16x8 xf[2][KSTEPS];
  float xx[2] = {0.0f, 0.0f};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int tok = t0 + 64 * wave + 32 * hh + l32;
    const uint16_t* xr = x + (xb + min(tok, N - 1)) * D + 8 * h2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      xf[hh][s] = *reinterpret_cast<const bf16x8*>(xr + 16 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)xf[hh][s][e];
        xx[hh] = fmaf(f, f, xx[hh]);
      }
    }
    xx[hh] += __shfl_xor(xx[hh], 32);
  }
  const int tiles = (C + BK - 1) / BK;
  const uint16_t* hib = chi + (size_t)bh * C * D;
  const uint16_t* lob = clo + (size_t)bh * C * D;
  const float* cnb = cnf + (size_t)bh * ((C + BK - 1) / BK * BK);
  auto issue = [&](int t) {
    unsigned char* buf = smem + (t & 1) * 2 * T::BYTES;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int p = 64 * (u * NW + wave) + lane;
      const int kr = p / T::KCPR;
      const size_t src = (size_t)min(t * BK + kr, C - 1) * D + T::kchunk(kr, p % T::KCPR) * 8;
      dma16(hib + src, buf + 1024 * (u * NW + wave));
      dma16(lob + src, buf + T::BYTES + 1024 * (u * NW + wave));
    }
    if (wave == 0 && lane < BK / 4) dma16(cnb + t * BK + 4 * lane, cns + (t & 1) * BK * 4);
  };
  int koff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = l32 * T::KROWB + (T::kchunk(l32, 2 * s + h2) << 4);
  float b1[2] = {INFINITY, INFINITY}, b2[2] = {INFINITY, INFINITY};
  int i1[2] = {C, C};
  issue(0);
  for (int t = 0; t < tiles; ++t) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile t landed
    __syncthreads();                     // every wave's copies landed; the other buffer is free
    if (t + 1 < tiles) issue(t + 1);
    const unsigned char* hb = smem + (t & 1) * 2 * T::BYTES;
    floatx16 acc[2][2];  // [tau][half]
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tau][hh][r] = 0.0f;
    // fragments [plane][tau] of k-step s, the next step's read ahead
    bf16x8 fa[2][2];
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        fa[pl][tau] = lds_read16(hb + pl * T::BYTES + tau * 32 * T::KROWB + koff[0]);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      bf16x8 fn[2][2];
      if (s + 1 < KSTEPS) {
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
            fn[pl][tau] = lds_read16(hb + pl * T::BYTES + tau * 32 * T::KROWB + koff[s + 1]);
      }
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            acc[tau][hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[pl][tau], xf[hh][s],
                                                                    acc[tau][hh], 0, 0, 0);
      if (s + 1 < KSTEPS) {
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau) fa[pl][tau] = fn[pl][tau];
      }
    }
    // lane: token l32 of each half, centroids t*64 + 32 tau + 8 (r / 4) + 4 h2 + r % 4
    // (+inf |c|^2 past C: such rows never win); the four |c|^2 of a register
    // group are read as one 16-byte fragment
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row0 = 32 * tau + 8 * q4 + 4 * h2;
        const float4 c4 = __builtin_bit_cast(float4, lds_read16(cns + ((t & 1) * BK + row0) * 4));
        const float cn4[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e, c = t * BK + row0 + e;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            // best two: b2 = median of (b1, b2, v) as b1 <= b2; b1 = min
            const float v = fmaf(-2.0f, acc[tau][hh][r], cn4[e]);
            const bool lt = v < b1[hh];
            b2[hh] = __builtin_amdgcn_fmed3f(b1[hh], b2[hh], v);
            b1[hh] = lt ? v : b1[hh];
            i1[hh] = lt ? c : i1[hh];
          }
        }
      }
  }
  const float cm = __uint_as_float(cmax_bits[bh]);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float p1 = b1[hh], p2 = b2[hh];
    int pi = i1[hh];
    {  // merge the two half-waves (the same token)
      const float o1 = __shfl_xor(p1, 32), o2 = __shfl_xor(p2, 32);
      const int oi = __shfl_xor(pi, 32);
      if (o1 < p1) {
        p2 = fminf(o2, p1);
        p1 = o1;
        pi = oi;
      } else if (o1 == p1) {
        p2 = p1;
        pi = min(pi, oi);
      } else {
        p2 = fminf(p2, o1);
      }
    }
    const int tok = t0 + 64 * wave + 32 * hh + l32;
    if (h2 == 0 && tok < N) {
      const float xn = sqrtf(xx[hh] * (1.0f + 1e-5f)) * (1.0f + 1e-6f);
      const float E = 1.25e-4f * xn * cm + 2.5e-7f * cm * cm;
      const bool sane = xn * cm < 1e30f && cm * cm < 1e30f && fabsf(p1) < 1e30f &&
                        fabsf(p2) < 1e30f;
      if (sane && p2 - p1 > 2.0f * E) {
        assign[xb + tok] = pi;
      } else {
        flag_list[xb + atomicAdd(&flag_cnt[bh], 1)] = tok;
      }
    }
  }
}

// (b) assign[t] for the listed tokens t of each (b, h), from float64
// distances. Workgroup (g, b, h) takes chunks g, g + G, ... of 16 listed
// tokens, its 4 waves a quarter of the centroids each: a wave holds the 16
// tokens in registers (lane: token lane % 16, channels 8 s + 2 (lane / 16) +
// 0..1) and takes its centroids 16 at a time, each lane loading the same
// channels of one centroid row (all its loads issued together, the next
// tile's while the current one multiplies); each lane keeps the best of its
// column of every 16 x 16 product for the 4 tokens it holds, the 16 lanes of
// a token group merge, then the 4 waves through LDS, smallest (distance,
// cluster) first, i.e. ties to the lower cluster. Every distance comes from
// the same float64 instruction sequence whichever tokens share its chunk.
constexpr int kExactGroups = 16;  // workgroups per (b, h) of km_exact_kernel

template <int D>
__global__ __launch_bounds__(256, 2) void km_exact_kernel(const uint16_t* __restrict__ x,
                                                          const double* __restrict__ cent,
                                                          const double* __restrict__ cnorm,
                                                          const int32_t* __restrict__ list,
                                                          const int32_t* __restrict__ list_cnt,
                                                          int32_t* __restrict__ assign, int N,
                                                          int C) {
  constexpr int CT = 16;  // centroids per step of a wave
  __shared__ double mb[4][16];
  __shared__ int mi[4][16];
  const int bh = blockIdx.y;
  const int th = threadIdx.x, lane = th & 63;
  const int wave = __builtin_amdgcn_readfirstlane(th >> 6);
  const int r = lane & 15, g = lane >> 4;
  const size_t xb = (size_t)bh * N;
  const int cnt = min(list_cnt[bh], N);
  const int32_t* lb = list + xb;
  const double* cb0 = cent + (size_t)bh * C * D;
  const double* cn0 = cnorm + (size_t)bh * C;
  // this wave's centroids: [c_lo, c_hi), a quarter of C in whole steps
  const int per = (C + 4 * CT - 1) / (4 * CT) * CT;
  const int c_lo = min(wave * per, C), c_hi = min(c_lo + per, C);
  auto load_tile = [&](int cb, double2(&y)[D / 8], double& cnc) {
    const int cr = min(cb + r, C - 1);
    const double* row = cb0 + (size_t)cr * D + 2 * g;
#pragma unroll
    for (int s = 0; s < D / 8; ++s) y[s] = *reinterpret_cast<const double2*>(row + 8 * s);
    cnc = cn0[cr];
  };
  for (int base = blockIdx.x * 16; base < cnt; base += gridDim.x * 16) {
    const int tok = lb[min(base + r, cnt - 1)];  // repeats past the count are not stored
    double2 xr[D / 8];
#pragma unroll
    for (int s = 0; s < D / 8; ++s) {
      const uint32_t two = *reinterpret_cast<const uint32_t*>(x + (xb + tok) * D + 8 * s + 2 * g);
      xr[s] = make_double2(bf16_f64((uint16_t)(two & 0xFFFFu)), bf16_f64((uint16_t)(two >> 16)));
    }
    double best[4] = {INFINITY, INFINITY, INFINITY, INFINITY};
    int bi[4] = {C, C, C, C};
    double2 y[D / 8];
    double cnc = 0.0;
    if (c_lo < c_hi) load_tile(c_lo, y, cnc);
    for (int cb = c_lo; cb < c_hi; cb += CT) {
      f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s = 0; s < D / 8; ++s) {
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[s].x, y[s].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[s].y, y[s].y, acc, 0, 0, 0);
      }
      const double cnu = cnc;
      if (cb + CT < c_hi) load_tile(cb + CT, y, cnc);
      // lane: tokens 4 e + g of the 16, centroid cb + r (increasing per lane)
      const int c = cb + r;
      if (c < c_hi) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double v = cnu - 2.0 * acc[e];
          if (v < best[e]) {
            best[e] = v;
            bi[e] = c;
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
      if (r == 0) {
        mb[wave][4 * e + g] = best[e];
        mi[wave][4 * e + g] = bi[e];
      }
    }
    __syncthreads();
    if (th < 16 && base + th < cnt) {
      double bv = mb[0][th];
      int bc = mi[0][th];
      for (int w = 1; w < 4; ++w) {
        const double ov = mb[w][th];
        const int oc = mi[w][th];
        if (ov < bv || (ov == bv && oc < bc)) {
          bv = ov;
          bc = oc;
        }
      }
      assign[xb + lb[base + th]] = min(bc, C - 1);  // (C only if no distance compared: NaN input)
    }
    __syncthreads();  // mb, mi are reused
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
  constexpr int U = 16;  // chunk counts in flight per lane (their loads issued together)
  int sum = 0;
  if (c < C)
    for (int cb = ch0; cb < ch1; cb += U) {
      int v[U];
#pragma unroll
      for (int x = 0; x < U; ++x) v[x] = cb + x < ch1 ? col[(size_t)(cb + x) * C] : 0;
#pragma unroll
      for (int x = 0; x < U; ++x) sum += v[x];
    }
  part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += part[w][lane];
  if (c < C) {
    for (int cb = ch0; cb < ch1; cb += U) {
      int v[U];
#pragma unroll
      for (int x = 0; x < U; ++x) v[x] = cb + x < ch1 ? col[(size_t)(cb + x) * C] : 0;
#pragma unroll
      for (int x = 0; x < U; ++x) {
        if (cb + x < ch1) col[(size_t)(cb + x) * C] = run;
        run += v[x];
      }
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
__global__ __launch_bounds__(D) void km_update_kernel(const uint16_t* __restrict__ x,
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
    // members in token order; eight rows in flight at a time, summed in order
    const int32_t* pm = perm + (size_t)bh * N + o0;
    const uint16_t* xh = x + (size_t)bh * N * D + t;
    double acc = 0.0;
    int m = 0;
    for (; m + 8 <= n; m += 8) {
      uint16_t xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = xh[(size_t)pm[m + e] * D];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += bf16_f64(xv[e]);
    }
    for (; m < n; ++m) acc += bf16_f64(xh[(size_t)pm[m] * D]);
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
// and of the key clusters (whole 16-key groups), the cluster of every query
// tile and the tile count. One workgroup per (b, h): exclusive scans of the
// per-cluster tile and group counts, 256 clusters at a time.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    before += i < w ? tmp[i] : 0;
    total += tmp[i];
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(256) void svg2_layout_kernel(
    const int32_t* __restrict__ qsize, const int32_t* __restrict__ ksize,
    int32_t* __restrict__ qpad_off, int32_t* __restrict__ kpad_off,
    int32_t* __restrict__ tile_cluster, int32_t* __restrict__ n_tiles, int Cq, int Ck, int BQ,
    int max_tiles) {
  __shared__ int tmp[4];
  const int bh = blockIdx.x, t = threadIdx.x;
  int tiles = 0;
  for (int c0 = 0; c0 < Cq; c0 += 256) {
    const int c = c0 + t;
    const int nt = c < Cq ? (qsize[(size_t)bh * Cq + c] + BQ - 1) / BQ : 0;
    int chunk_total;
    const int first = tiles + block_exclusive_scan(nt, tmp, chunk_total);
    if (c < Cq) {
      qpad_off[(size_t)bh * Cq + c] = first * BQ;
      for (int u = 0; u < nt; ++u) tile_cluster[(size_t)bh * max_tiles + first + u] = c;
    }
    tiles += chunk_total;
  }
  if (t == 0) n_tiles[bh] = tiles;
  int groups = 0;
  for (int c0 = 0; c0 < Ck; c0 += 256) {
    const int c = c0 + t;
    const int ng = c < Ck ? (ksize[(size_t)bh * Ck + c] + 15) / 16 : 0;
    int chunk_total;
    const int first = groups + block_exclusive_scan(ng, tmp, chunk_total);
    if (c < Ck) kpad_off[(size_t)bh * Ck + c] = first * 16;
    groups += chunk_total;
  }
}

// Per (b, h, query cluster), one wave: the 16-key groups of its selected key
// clusters, in the selection's order, as entries 32 * group + (valid keys of
// the group); the list is padded to whole 64-key chunks (four entries) with
// entries of no valid key, and list_cnt holds the chunk count. The selected
// clusters are taken 64 at a time, one per lane, placed by a wave scan of
// their group counts.
__global__ __launch_bounds__(256) void svg2_lists_kernel(const int32_t* __restrict__ sidx,
                                                         const int32_t* __restrict__ scnt,
                                                         const int32_t* __restrict__ kpad_off,
                                                         const int32_t* __restrict__ ksize,
                                                         int32_t* __restrict__ lists,
                                                         int32_t* __restrict__ list_cnt, int Cq,
                                                         int Ck, int max_list, size_t rows) {
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const size_t bh = row / Cq;
  const int cnt = scnt[row];
  int32_t* out = lists + row * max_list;
  int pos = 0;
  for (int e0 = 0; e0 < cnt; e0 += 64) {
    const int e = e0 + lane;
    int n = 0, base = 0;
    if (e < cnt) {
      const int j = sidx[row * Ck + e];
      n = ksize[bh * Ck + j];
      base = kpad_off[bh * Ck + j] / 16;
    }
    const int ng = (n + 15) / 16;
    int x = ng;  // inclusive scan of the group counts over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    const int first = pos + x - ng;
    for (int u = 0; u < ng; ++u) out[first + u] = (base + u) * 32 + min(16, n - 16 * u);
    pos += __shfl(x, 63);
  }
  const int padded = (pos + 3) & ~3;
  if (lane < padded - pos) out[pos + lane] = 0;  // group 0 (finite data), no valid key
  if (lane == 0) list_cnt[row] = padded / 4;
}

// Dispatch order of the attention's query tiles. Tiles carry very different
// work (a query cluster keeps anywhere from one to several hundred 64-key
// chunks), and workgroups go round-robin to the 8 XCDs, so slot i of XCD x
// is workgroup 8 i + x (the positions xcd_remap gives). Every XCD receives a
// contiguous, head-major range of the real tiles holding an eighth of the
// total work (weight = chunks + kTileCost for a tile's fixed cost), clamped
// so that no XCD gets more tiles than it has slots, and runs that range
// heaviest tile first, so the range ends on short tiles instead of a long
// one started late. Entries are b h * max_tiles + tile, -1 for unused slots.
// One workgroup per XCD; thread t walks grid entries [t R, t R + R) three
// times (weights and ranks, histogram, placement). The placement takes its
// slots with LDS atomics, so the order among tiles of equal weight can vary
// from call to call; every tile's output is computed the same way in any
// order.
constexpr int kTileCost = 3;
constexpr int kOrderBins = 1024;

__global__ __launch_bounds__(1024) void svg2_order_kernel(const int32_t* __restrict__ n_tiles,
                                                          const int32_t* __restrict__ tile_cluster,
                                                          const int32_t* __restrict__ list_cnt,
                                                          int32_t* __restrict__ order, int BH,
                                                          int Cq, int max_tiles) {
  __shared__ long long wred[16];
  __shared__ int cred[16];
  __shared__ int h8[8];
  __shared__ int bins[kOrderBins];
  __shared__ int range[2];
  constexpr int XCDS = 8;
  const int x = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int total = BH * max_tiles;
  const int R = (total + 1023) / 1024;
  const int g0 = min(t * R, total), g1 = min(g0 + R, total);
  auto weight = [&](int g) -> int {  // 0 for slots past a head's tiles
    const int bh = g / max_tiles, tl = g % max_tiles;
    if (tl >= min(n_tiles[bh], max_tiles)) return 0;
    return max(list_cnt[(size_t)bh * Cq + tile_cluster[g]], 0) + kTileCost;
  };
  long long wsum = 0;
  int vcnt = 0;
  for (int g = g0; g < g1; ++g) {
    const int wt = weight(g);
    wsum += wt;
    vcnt += wt > 0;
  }
  // exclusive scans of the work and of the tile count over the threads
  long long ws = wsum;
  int vs = vcnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long a = __shfl_up(ws, off);
    const int b = __shfl_up(vs, off);
    if (lane >= off) { ws += a; vs += b; }
  }
  if (lane == 63) { wred[w] = ws; cred[w] = vs; }
  if (t < 8) h8[t] = 0;
  for (int i = t; i < kOrderBins; i += 1024) bins[i] = 0;
  __syncthreads();
  long long wbase = 0, W = 0;
  int rbase = 0, T = 0;
  for (int i = 0; i < 16; ++i) {
    wbase += i < w ? wred[i] : 0;
    rbase += i < w ? cred[i] : 0;
    W += wred[i];
    T += cred[i];
  }
  wbase += ws - wsum;
  rbase += vs - vcnt;
  // tiles whose work starts in the k-th eighth of the total
  {
    long long p = wbase;
    for (int g = g0; g < g1; ++g) {
      const int wt = weight(g);
      if (wt > 0) atomicAdd(&h8[(int)min(8 * p / max(W, 1ll), 7ll)], 1);
      p += wt;
    }
  }
  __syncthreads();
  const int per = total / XCDS, rem = total % XCDS;
  auto cap = [&](int y) { return per + (y < rem ? 1 : 0); };
  if (t == 0) {
    int s = 0, cut = 0, after = total;  // after: slots of XCDs y.. ; cut: tiles before eighth y+1
    for (int y = 0; y < XCDS; ++y) {
      cut += h8[y];
      after -= cap(y);
      const int lo = max(s, T - after), hi = min(s + cap(y), T);
      const int e = min(max(y == XCDS - 1 ? T : cut, lo), hi);
      if (y == x) { range[0] = s; range[1] = e; }
      s = e;
    }
  }
  __syncthreads();
  const int s0 = range[0], s1 = range[1];
  auto bin_of = [](int wt) { return kOrderBins - 1 - min(wt, kOrderBins - 1); };  // heaviest first
  {
    int r = rbase;
    for (int g = g0; g < g1; ++g) {
      const int wt = weight(g);
      if (wt > 0) {
        if (r >= s0 && r < s1) atomicAdd(&bins[bin_of(wt)], 1);
        ++r;
      }
    }
  }
  __syncthreads();
  {  // exclusive scan of the bins (one per thread)
    const int v = t < kOrderBins ? bins[t] : 0;
    int xs = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(xs, off);
      if (lane >= off) xs += y;
    }
    __syncthreads();
    if (lane == 63) cred[w] = xs;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += cred[i];
    if (t < kOrderBins) bins[t] = before + xs - v;
  }
  __syncthreads();
  const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  {
    int r = rbase;
    for (int g = g0; g < g1; ++g) {
      const int wt = weight(g);
      if (wt > 0) {
        if (r >= s0 && r < s1) order[base + atomicAdd(&bins[bin_of(wt)], 1)] = g;
        ++r;
      }
    }
  }
  for (int j = s1 - s0 + t; j < cap(x); j += 1024) order[base + j] = -1;
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
// The variable-size clusters without padding to whole tiles on the key side
// ("Sparse VideoGen2" page, section 2C: sparse loading of the scattered keys
// and values, dense compute on contiguous queries). Key clusters are padded
// only to whole 16-key groups; a query cluster's list names the groups of its
// kept key clusters, four to a 64-key chunk. One workgroup per padded query
// tile (BQ rows of one cluster), BQ/32 waves of 32 queries (rows past the
// cluster's end are zero and their results are not stored), taken in the
// order svg2_order_kernel set: work-balanced XCD ranges, heaviest tile
// first. Every chunk's K rows and packed V^T slots are gathered group by group
// global -> LDS by direct-to-LDS copies with per-lane source addresses (K:
// one group per copy instruction and wave; V^T: the two 16-byte halves of a
// group's slots in every channel row), into the tile layouts of the sparse
// kernel. The loop is the sparse kernel's: the S^T product of chunk it+1 is
// issued during the softmax and P V of chunk it, K tiles and V^T tiles are
// double-buffered one chunk apart, the running maximum is raised lazily, and
// a chunk's keys past their group's valid count get -inf. Rows go back to
// their tokens.
// (D = 128 with BQ = 64 holds one wave per SIMD: two workgroups of two waves
// fill a CU's LDS)
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, (D == 128 && BQ == 64) ? 1 : 2) void svg2_attn_kernel(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vtp, const int32_t* __restrict__ tile_cluster,
    const int32_t* __restrict__ tile_order, const int32_t* __restrict__ lists,
    const int32_t* __restrict__ list_cnt, const int32_t* __restrict__ perm_q,
    const int32_t* __restrict__ off_q, const int32_t* __restrict__ size_q,
    const int32_t* __restrict__ qpad_off, uint16_t* __restrict__ o, int N, int NQP, int NKP,
    int Cq, int max_tiles, int max_list, int n_ktiles, float c) {
  constexpr int NW = BQ / 32;
  using T = Tile<D>;
  constexpr int LOADS = BK * D / 8 / 64 / NW;
  constexpr int DT = D / 32, KSTEPS = D / 16, HALF = KSTEPS / 2;
  constexpr float kRescale = 8.0f;  // raise the running maximum only past 2^8 (P <= 2^8)
  __shared__ __align__(16) unsigned char smem[4 * T::BYTES];
  unsigned char* const kbuf = smem;
  unsigned char* const vbuf = smem + 2 * T::BYTES;

  const int enc = tile_order[xcd_remap(blockIdx.x, (int)gridDim.x)];
  if (enc < 0) return;
  const int bh = enc / max_tiles, tile = enc % max_tiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int cq = tile_cluster[(size_t)bh * max_tiles + tile];
  const int qsz = size_q[(size_t)bh * Cq + cq];
  const int local = tile * BQ - qpad_off[(size_t)bh * Cq + cq] + wave * 32 + l32;
  // a wave whose 32 rows all lie past the cluster's end only copies its share
  // of the tiles and passes the barriers; its SIMD's matrix core and VALU are
  // left to the other workgroup's wave
  const bool idle = __builtin_amdgcn_readfirstlane(local - l32) >= qsz;
  const int prow = tile * BQ + wave * 32 + l32;  // row of the padded permuted Q

  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qr = qp + ((size_t)bh * NQP + prow) * D + 8 * h2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
  }
  const size_t lrow = (size_t)bh * Cq + cq;
  const int count = min(max(list_cnt[lrow], 0), max_list / 4);
  const int32_t* ents = lists + lrow * max_list;
  const int gmax = n_ktiles * 4 - 1;  // last valid group index
  // the four entries of chunk i sit in lanes 0..3 of one register, loaded two
  // steps before their first use
  auto load_ent = [&](int i) { return i < count && lane < 4 ? ents[4 * i + lane] : 0; };
  auto gid_of = [&](int e) { return min(max(e >> 5, 0), gmax); };

  const char* kh = reinterpret_cast<const char*>(kp + (size_t)bh * NKP * D);
  const char* vh = reinterpret_cast<const char*>(vtp + (size_t)bh * n_ktiles * D * BK);
  // Copy u of this wave covers tile positions p = p0 + 64 NW u. K: row
  // kr = p / KCPR, i.e. row kr mod 16 of group kgroup(u) (one group for the
  // whole wave). V^T: channel row vr = p / 8 and logical chunk sc, the 16-byte
  // half sc mod 2 of group sc / 2's slots (the lane's own group). The lane's
  // parts that do not depend on u are computed once: the swizzles see u only
  // through multiples of their period.
  const int p0 = 64 * wave + lane;
  constexpr int KRU = 64 * NW / T::KCPR;  // K rows per copy step
  const int kr0 = p0 / T::KCPR, kc0 = p0 % T::KCPR;
  auto kl = [&](int u) {
    const int kr = kr0 + KRU * u;
    return (uint32_t)(((kr & 15) * D + T::kchunk(kr, kc0) * 8) * 2);
  };
  const int vr0 = p0 / T::VCPR, vsc = T::vchunk(vr0, p0 % T::VCPR), vgrp = vsc >> 1;
  const uint32_t vl0 = (uint32_t)((vr0 * BK + (vsc & 1) * 8) * 2);
  auto kgroup = [&](int u) { return (64 * (u * NW + wave)) / (16 * T::KCPR); };
  // byte offsets (within the head) of K copy u and V^T copy u for a chunk
  // whose entries are in e (lanes 0..3)
  auto koff_of = [&](int e, int u) {
    const int gid = gid_of(__builtin_amdgcn_readlane(e, kgroup(u)));
    return (uint32_t)gid * (16 * D * 2) + kl(u);
  };
  auto vsel = [&](int e) {  // this lane's group: tile and slot offset
    uint32_t t = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int gid = gid_of(__builtin_amdgcn_readlane(e, g));
      const uint32_t tg = (uint32_t)((gid >> 2) * D * BK * 2 + (gid & 3) * 32);
      t = vgrp == g ? tg : t;
    }
    return t + vl0;
  };
  auto voff_of = [&](uint32_t vs, int u) { return vs + (uint32_t)(8 * NW * u * BK * 2); };
  auto stageK = [&](int e, int b) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      dma16(kh + koff_of(e, u), kbuf + b * T::BYTES + 1024 * (u * NW + wave));
  };
  auto stageV = [&](int e, int b) {
    const uint32_t vs = vsel(e);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      dma16(vh + voff_of(vs, u), vbuf + b * T::BYTES + 1024 * (u * NW + wave));
  };

  int koff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = l32 * T::KROWB + (T::kchunk(l32, 2 * s + h2) << 4);
  int voff[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) voff[g] = l32 * T::VROWB + (T::vchunk(l32, 2 * g + h2) << 4);

  // k-steps [S0, S1) of S^T = K Q^T from the K tile at kb
  auto qk = [&](const unsigned char* kb, floatx16(&st)[2], int S0, int S1, auto&& hook) {
    bf16x8 ka[2] = {lds_read16(kb + koff[S0]), lds_read16(kb + 32 * T::KROWB + koff[S0])};
#pragma unroll
    for (int s = S0; s < S1; ++s) {
      hook(s - S0);
      bf16x8 kn[2];
      if (s + 1 < S1) {
        kn[0] = lds_read16(kb + koff[s + 1]);
        kn[1] = lds_read16(kb + 32 * T::KROWB + koff[s + 1]);
      }
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        st[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[tau], qf[s], st[tau], 0, 0, 0);
      if (s + 1 < S1) { ka[0] = kn[0]; ka[1] = kn[1]; }
    }
  };

  floatx16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;
  auto zero_s = [&](floatx16(&st)[2]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[tau][r] = 0.0f;
  };
  // keys past their group's valid count get -inf; group g of the chunk is
  // registers 8 (g & 1) .. + 7 of S^T tile g / 2, and most groups are full,
  // so only a partial group's registers are touched (a uniform branch each)
  auto mask_s = [&](floatx16(&st)[2], int e) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int val = __builtin_amdgcn_readlane(e, g) & 31;
      if (val < 16) {
#pragma unroll
        for (int r8 = 0; r8 < 8; ++r8) {
          const int r = 8 * (g & 1) + r8;
          const int within = 8 * (r8 >> 2) + 4 * h2 + (r8 & 3);
          if (within >= val) st[g >> 1][r] = -INFINITY;
        }
      }
    }
  };
  floatx16 sc[2], sn[2];  // S^T of the current and the next chunk
  // entries of chunks it, it+1, it+2 (and it+3 in flight)
  int e0 = load_ent(0), e1 = load_ent(1), e2 = load_ent(2);
  zero_s(sc);
  if (count > 0) {
    stageK(e0, 0);
    stageV(e0, 0);
    if (count > 1) stageK(e1, 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (!idle) qk(kbuf, sc, 0, KSTEPS, [](int) {});
  }

  // one chunk: softmax and P V of chunk it (S^T in sc), and with NEXT the
  // S^T of chunk it+1 into sn, interleaved with the copies for later steps
  auto step = [&](int it, auto next_tag, floatx16(&sc)[2], floatx16(&sn)[2]) {
    constexpr bool NEXT = decltype(next_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K of it+1, V^T of it, entries landed
    __syncthreads();                     // and every wave is done with step it-1's buffers
    const int e3 = load_ent(it + 3);
    unsigned char* kdst = kbuf + (it & 1) * T::BYTES;         // K of chunk it+2
    unsigned char* vdst = vbuf + ((it + 1) & 1) * T::BYTES;   // V^T of chunk it+1
    const int ek = it + 2 < count ? e2 : e1;  // a repeat of it+1 when there is none (not read)
    uint32_t vs = 0;
    if constexpr (NEXT) vs = vsel(e1);
    auto kdma = [&](int sl) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        if (u * HALF / LOADS == sl) dma16(kh + koff_of(ek, u), kdst + 1024 * (u * NW + wave));
    };
    auto vdma = [&](int sl) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        if (u * HALF / LOADS == sl) dma16(vh + voff_of(vs, u), vdst + 1024 * (u * NW + wave));
    };
    const unsigned char* kn = kbuf + ((it + 1) & 1) * T::BYTES;
    const unsigned char* vb = vbuf + (it & 1) * T::BYTES;
    {
      if constexpr (NEXT) {
        zero_s(sn);
        qk(kn, sn, 0, HALF, kdma);
      }

      mask_s(sc, e0);
      float mloc = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sc[tau][r]);
      mloc = pair_max(mloc);
      if (__any((mloc - m) * c > kRescale)) {
        const float m_new = fmaxf(m, mloc);
        const float alpha_r = m_new > -INFINITY ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.0f;
        m = m_new;
        lsum *= alpha_r;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha_r;
      }

      if constexpr (NEXT) qk(kn, sn, HALF, KSTEPS, vdma);
      // a row with no valid key yet (m = -inf) gives P = 0
      const float mc = m > -INFINITY ? m * c : 0.0f;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[tau][r] = __builtin_amdgcn_exp2f(fmaf(sc[tau][r], c, -mc));

      bf16x8 va[DT];
#pragma unroll
      for (int i = 0; i < DT; ++i) va[i] = lds_read16(vb + i * 32 * T::VROWB + voff[0]);
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const int tau = G >> 1, hk = G & 1;
        const bf16x8 pb = pack_bf16x8(sc[tau], 8 * hk);
        lsum = row_sum_bf16x8(pb, lsum);
        bf16x8 vn[DT];
        if (G + 1 < 4) {
#pragma unroll
          for (int i = 0; i < DT; ++i) vn[i] = lds_read16(vb + i * 32 * T::VROWB + voff[G + 1]);
        }
#pragma unroll
        for (int i = 0; i < DT; ++i)
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb, oacc[i], 0, 0, 0);
        if (G + 1 < 4) {
#pragma unroll
          for (int i = 0; i < DT; ++i) va[i] = vn[i];
        }
      }
    }
    e0 = e1;
    e1 = e2;
    e2 = e3;
  };
  if (idle) {  // the same barriers and copies, no products
    for (int it = 0; it < count; ++it) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int e3 = load_ent(it + 3);
      if (it + 1 < count) {
        unsigned char* kdst = kbuf + (it & 1) * T::BYTES;
        unsigned char* vdst = vbuf + ((it + 1) & 1) * T::BYTES;
        const int ek = it + 2 < count ? e2 : e1;
        const uint32_t vs = vsel(e1);
#pragma unroll
        for (int u = 0; u < LOADS; ++u) dma16(kh + koff_of(ek, u), kdst + 1024 * (u * NW + wave));
#pragma unroll
        for (int u = 0; u < LOADS; ++u) dma16(vh + voff_of(vs, u), vdst + 1024 * (u * NW + wave));
      }
      e0 = e1;
      e1 = e2;
      e2 = e3;
    }
  } else {
    int it = 0;
    for (; it + 2 < count; it += 2) {
      step(it, std::true_type{}, sc, sn);
      step(it + 1, std::true_type{}, sn, sc);
    }
    if (it + 1 < count) {
      step(it, std::true_type{}, sc, sn);
      step(it + 1, std::false_type{}, sn, sc);
    } else if (it < count) {
      step(it, std::false_type{}, sc, sn);
    }
  }

  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (local < qsz) {
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

// Token pairs per (b, h): useful = sum over query clusters of |cluster| times
// the tokens of its kept key clusters; computed = the pairs the attention
// kernel evaluates, BQ rows per query tile times 64 keys per listed chunk.
__global__ __launch_bounds__(256) void svg2_pairs_kernel(
    const int32_t* __restrict__ sidx, const int32_t* __restrict__ scnt,
    const int32_t* __restrict__ size_q, const int32_t* __restrict__ size_k,
    const int32_t* __restrict__ list_cnt, unsigned long long* __restrict__ counts, int Cq,
    int Ck, int BQ) {
  __shared__ unsigned long long acc[2];
  const int bh = blockIdx.x;
  if (threadIdx.x < 2) acc[threadIdx.x] = 0ull;
  __syncthreads();
  unsigned long long useful = 0, computed = 0;
  for (int cq = threadIdx.x; cq < Cq; cq += 256) {
    const size_t row = (size_t)bh * Cq + cq;
    const long long nq = size_q[row];
    long long keys = 0;
    for (int e = 0; e < scnt[row]; ++e) keys += size_k[(size_t)bh * Ck + sidx[row * Ck + e]];
    useful += (unsigned long long)(nq * keys);
    computed += (unsigned long long)(BQ * ((nq + BQ - 1) / BQ)) * 64ull * (unsigned)list_cnt[row];
  }
  atomicAdd(&acc[0], useful);
  atomicAdd(&acc[1], computed);
  __syncthreads();
  if (threadIdx.x < 2) counts[2 * (size_t)bh + threadIdx.x] = acc[threadIdx.x];
}

// --------------------------------------------------------------- driver
template <int D>
hipError_t kmeans_run(const Svg2Launch& a, const uint16_t* x, int C, double* cent, double* cnorm,
                      int32_t* assign, int32_t* size, int32_t* off, int32_t* perm, hipStream_t s) {
  const int BH = a.B * a.H, nch = (a.N + 63) / 64;
  const size_t rows = (size_t)BH * a.N, chunks = (size_t)BH * nch, cc = chunks * C;
  uint32_t* cmax_bits = reinterpret_cast<uint32_t*>(a.kaux);
  int32_t* flag_cnt = a.kaux + BH;
  hipLaunchKernelGGL((km_init_kernel<D>), dim3(C, BH), dim3(D), 0, s, x, cent, cnorm, a.N, C);
  for (int it = 0; it <= a.iters; ++it) {
    hipLaunchKernelGGL(fill_i32_zero_kernel, dim3(1), dim3(256), 0, s, a.kaux, (size_t)2 * BH);
    hipLaunchKernelGGL((km_planes_kernel<D>), dim3((C + kPlaneClusters - 1) / kPlaneClusters, BH),
                       dim3(256), 0, s, cent, cnorm, a.chi, a.clo, a.cnf, cmax_bits, C);
    hipLaunchKernelGGL((km_filter_kernel<D>), dim3((a.N + 255) / 256, BH), dim3(256), 0, s, x,
                       a.chi, a.clo, a.cnf, cmax_bits, assign, a.kflags, flag_cnt, a.N, C);
    hipLaunchKernelGGL((km_exact_kernel<D>), dim3(kExactGroups, BH), dim3(256), 0, s, x, cent,
                       cnorm, a.kflags, flag_cnt, assign, a.N, C);
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
  const int NQP = a.max_tiles * BQ, NKP = a.n_ktiles * BK;
  if (a.phase == kSvg2Attend) {
    hipLaunchKernelGGL((svg2_attn_kernel<D, BQ>), dim3(BH * a.max_tiles), dim3(BQ * 2), 0, s, a.qp,
                       a.kp, a.vtp, a.tile_cluster, a.tile_order, a.lists, a.list_cnt, a.perm_q,
                       a.off_q, a.size_q, a.qpad_off, a.o, a.N, NQP, NKP, a.Cq, a.max_tiles,
                       a.max_list, a.n_ktiles, a.scale * 1.4426950408889634f);
    return hipGetLastError();
  }
  hipError_t e = kmeans_run<D>(a, a.q, a.Cq, a.centq, a.normq, a.assign_q, a.size_q, a.off_q,
                               a.perm_q, s);
  if (e == hipSuccess)
    e = kmeans_run<D>(a, a.k, a.Ck, a.centk, a.normk, a.assign_k, a.size_k, a.off_k, a.perm_k, s);
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
  // padded layouts, group lists, gathers
  hipLaunchKernelGGL(svg2_layout_kernel, dim3(BH), dim3(256), 0, s, a.size_q, a.size_k,
                     a.qpad_off, a.kpad_off, a.tile_cluster, a.n_tiles, a.Cq, a.Ck, BQ,
                     a.max_tiles);
  const size_t lrows = (size_t)BH * a.Cq;
  hipLaunchKernelGGL(svg2_lists_kernel, dim3((unsigned)((lrows + 3) / 4)), dim3(256), 0, s, a.sidx,
                     a.scnt, a.kpad_off, a.size_k, a.lists, a.list_cnt, a.Cq, a.Ck, a.max_list,
                     lrows);
  hipLaunchKernelGGL(svg2_order_kernel, dim3(8), dim3(1024), 0, s, a.n_tiles, a.tile_cluster,
                     a.list_cnt, a.tile_order, BH, a.Cq, a.max_tiles);
  hipLaunchKernelGGL((svg2_gather_kernel<D>), dim3(a.Cq, BH), dim3(256), 0, s, a.q, a.perm_q,
                     a.off_q, a.size_q, a.qpad_off, a.qp, a.N, a.Cq, BQ, NQP);
  hipLaunchKernelGGL((svg2_gather_kernel<D>), dim3(a.Ck, BH), dim3(256), 0, s, a.k, a.perm_k,
                     a.off_k, a.size_k, a.kpad_off, a.kp, a.N, a.Ck, 16, NKP);
  hipLaunchKernelGGL((svg2_gather_kernel<D>), dim3(a.Ck, BH), dim3(256), 0, s, a.v, a.perm_k,
                     a.off_k, a.size_k, a.kpad_off, a.vp, a.N, a.Ck, 16, NKP);
  hipLaunchKernelGGL((pack_kernel<D>), dim3(a.n_ktiles, BH), dim3(2 * D), 0, s, a.vp, a.vtp,
                     NKP, a.n_ktiles);
  if (a.phase == kSvg2Cluster) return hipGetLastError();
  hipLaunchKernelGGL((svg2_attn_kernel<D, BQ>), dim3(BH * a.max_tiles), dim3(BQ * 2), 0, s, a.qp,
                     a.kp, a.vtp, a.tile_cluster, a.tile_order, a.lists, a.list_cnt, a.perm_q,
                     a.off_q, a.size_q, a.qpad_off, a.o, a.N, NQP, NKP, a.Cq, a.max_tiles,
                     a.max_list, a.n_ktiles, a.scale * 1.4426950408889634f);
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
  a.max_groups = (int)((N + 15) / 16 + a.Ck);
  a.n_ktiles = (a.max_groups + 3) / 4;
  a.max_list = 4 * a.n_ktiles;
  const size_t NQP = (size_t)a.max_tiles * a.block_q, NKP = (size_t)a.n_ktiles * BK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = w ? w + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  a.chi = reinterpret_cast<uint16_t*>(take(BH * Cm * d * 2));
  a.clo = reinterpret_cast<uint16_t*>(take(BH * Cm * d * 2));
  a.cnf = reinterpret_cast<float*>(take(BH * ((Cm + BK - 1) / BK * BK) * 4));
  a.kaux = reinterpret_cast<int32_t*>(take(BH * 2 * 4));
  a.kflags = reinterpret_cast<int32_t*>(take(BH * N * 4));
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
  a.n_tiles = reinterpret_cast<int32_t*>(take(BH * 4));
  a.tile_order = reinterpret_cast<int32_t*>(take(BH * a.max_tiles * 4));
  a.lists = reinterpret_cast<int32_t*>(take(BH * a.Cq * a.max_list * 4));
  a.list_cnt = reinterpret_cast<int32_t*>(take(BH * a.Cq * 4));
  a.qp = reinterpret_cast<uint16_t*>(take(BH * NQP * d * 2));
  a.kp = reinterpret_cast<uint16_t*>(take(BH * NKP * d * 2));
  a.vp = reinterpret_cast<uint16_t*>(take(BH * NKP * d * 2));
  a.vtp = reinterpret_cast<uint16_t*>(take(BH * NKP * d * 2));
  return off;
}

hipError_t launch_svg2_pairs(const Svg2Launch& a, unsigned long long* counts, hipStream_t s) {
  hipLaunchKernelGGL(svg2_pairs_kernel, dim3(a.B * a.H), dim3(256), 0, s, a.sidx, a.scnt,
                     a.size_q, a.size_k, a.list_cnt, counts, a.Cq, a.Ck, a.block_q);
  return hipGetLastError();
}

hipError_t launch_svg2(const Svg2Launch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_svg2_t<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_svg2_t<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_svg2_t<64, 128>(a, s);
  return launch_svg2_t<64, 64>(a, s);
}

}  // namespace sparge
