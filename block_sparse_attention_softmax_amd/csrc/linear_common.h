// Linear-branch code of the forward and the backward translation units: the
// per-head branch flags (post-tuning branch dropping), the totals
// H_tot = sum_u phi(K_u)^T V_u, z_tot = sum_u phi(K_u), and (for the
// backward) a query block's H_D, z_D over its dropped blocks.
#pragma once

#include "internal.h"
#include "tiles.h"

namespace sparge {
namespace {

// ------------------------------------------------ H_D, z_D of a query block
constexpr int kMaxLinKeyBlocks = 4096;  // capacity of the per-row kept bitmap
// query blocks per (b, h) of the linear branch: block_q = d >= block_k, so n_q <= n_k <= 4096
constexpr int kMaxLinQueryBlocks = 4096;

// LDS of form_hd: four stages of (phi(K)^T, V^T) tiles, the complement list
// and the bitmap; H_D (rows of HP floats) and z_D overlay the stages at the
// end, and the backward's per-row part (phi(Q), dnum rows) follows them.
template <int D>
struct LinRowsLds {
  static constexpr int HP = D + 4, FP = D + 4, CH = 32, TILE = D * BK * 2;
  // part one: four stages of (phi(K)^T, V^T); part two reuses the space
  static constexpr int STAGE = 2 * TILE, NBUF = 4, BUFS = NBUF * STAGE;
  static constexpr int HS = 0, ZS = HS + D * HP * 4, FQ = ZS + D * 4, DN = FQ + CH * FP * 4,
                       DDEN = DN + CH * FP * 4, PART2 = DDEN + CH * 4;
  static constexpr int LIST = (BUFS > PART2 ? BUFS : PART2), BITS = LIST + kMaxLinKeyBlocks / 2 * 4,
                       BYTES = BITS + kMaxLinKeyBlocks / 8;
};

// H_D = sum over the key blocks that a query block does not list of
// phi(K_j)^T V_j (d x d, row = phi(K) channel) and z_D = sum phi(K_j), into
// LDS (Hs at LinRowsLds::HS with rows of HP floats, zs at ZS), on the matrix
// cores from the packed phi(K)^T and V^T tiles of whichever list is shorter:
// H_tot minus the listed blocks, or the blocks not listed (a bitmap of the
// list, then wave 0 writes the complement in increasing order; with more key
// blocks than the bitmap holds, always the listed blocks). The tiles are
// copied global -> LDS by direct-to-LDS loads three blocks ahead of their
// products (four buffers behind a fence-free barrier, each wave waiting for
// exactly the copies the next block reads). Called by all 256 threads of the
// workgroup; ends with a barrier after Hs and zs are written.
template <int D>
__device__ __forceinline__ void form_hd(unsigned char* smem, const uint16_t* __restrict__ phikt,
                                        const uint16_t* __restrict__ vt,
                                        const float* __restrict__ lin_h,
                                        const float* __restrict__ lin_z,
                                        const int32_t* __restrict__ ids, int count, int bh,
                                        int n_k) {
  using T = Tile<D>;
  using LS = LinRowsLds<D>;
  constexpr int DT = D / 32, HP = LS::HP, NTILE = DT * DT, TPW = (NTILE + 3) / 4;
  constexpr int VU = D * T::VCPR / 256;  // 16-byte copies per thread and tile
  float* const Hs = reinterpret_cast<float*>(smem + LS::HS);
  float* const zs = reinterpret_cast<float*>(smem + LS::ZS);
  int32_t* const clist = reinterpret_cast<int32_t*>(smem + LS::LIST);
  uint32_t* const kept_bits = reinterpret_cast<uint32_t*>(smem + LS::BITS);
  const int th = threadIdx.x, lane = th & 63;
  const int wave = __builtin_amdgcn_readfirstlane(th >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;

  const bool bitmap = n_k <= kMaxLinKeyBlocks;  // else the listed blocks, always
  const int words = bitmap ? (n_k + 31) / 32 : 0;
  for (int w = th; w < words; w += 256) kept_bits[w] = 0u;
  __syncthreads();
  if (bitmap)
    for (int e = th; e < count; e += 256) {
      const int j = min(max(ids[e], 0), n_k - 1);
      atomicOr(&kept_bits[j >> 5], 1u << (j & 31));
    }
  __syncthreads();
  // wave 0 lists the blocks not listed in increasing order (at most CAP of
  // them) and counts them; that list is used when it is the shorter one
  constexpr int CAP = kMaxLinKeyBlocks / 2 - 1;  // clist[CAP] holds the count
  if (wave == 0) {
    int base = 0;
    for (int w0 = 0; w0 < words; w0 += 64) {
      const int w = w0 + lane;
      uint32_t inv = 0u;
      if (w < words) {
        inv = ~kept_bits[w];
        if (32 * w + 32 > n_k) inv &= (1u << (n_k - 32 * w)) - 1u;
      }
      const int c1 = __popc(inv);
      int incl = c1;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int pos = base + incl - c1;
      while (inv) {
        if (pos < CAP) clist[pos] = 32 * w + __ffs(inv) - 1;
        ++pos;
        inv &= inv - 1u;
      }
      base += __shfl(incl, 63);
    }
    if (lane == 0) clist[CAP] = bitmap ? base : CAP + 1;
  }
  __syncthreads();
  const int n_off = __builtin_amdgcn_readfirstlane(clist[CAP]);
  const bool use_kept = !(n_off < count && n_off <= CAP);
  const int L = use_kept ? count : n_off;
  auto blk = [&](int e) {
    return use_kept ? min(max(ids[e], 0), n_k - 1) : __builtin_amdgcn_readfirstlane(clist[e]);
  };
  uint32_t vofs[VU];  // per-thread source offsets (elements) of the tile copies
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = u * 256 + th, r = p / T::VCPR;
    vofs[u] = (uint32_t)(r * BK + T::vchunk(r, p % T::VCPR) * 8);
  }
  const size_t vtile = (size_t)D * BK;
  auto issue = [&](int j, int b) {  // 2 VU copies per thread, the same for every wave
    const uint16_t* pk = phikt + ((size_t)bh * n_k + j) * vtile;
    const uint16_t* pv = vt + ((size_t)bh * n_k + j) * vtile;
    unsigned char* dst = smem + b * LS::STAGE + (wave * 64) * 16;
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      dma16(pk + vofs[u], dst + u * 256 * 16);
      dma16(pv + vofs[u], dst + LS::TILE + u * 256 * 16);
    }
  };
  floatx16 acc[TPW];
  float zp[TPW];
#pragma unroll
  for (int s2 = 0; s2 < TPW; ++s2) {
    zp[s2] = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s2][r] = 0.0f;
  }
  const int pre = min(L, LS::NBUF - 1);
  for (int e = 0; e < pre; ++e) issue(blk(e), e);
  for (int e = 0; e < L; ++e) {
    const int ahead = min(L - 1 - e, LS::NBUF - 2);  // later blocks already in flight
    static_assert(2 * VU * (LS::NBUF - 2) <= 63, "vmcnt range");
    if (ahead >= 2)
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * VU) & 15) | (((4 * VU) >> 4) << 14));
    else if (ahead == 1)
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * VU) & 15) | (((2 * VU) >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    barrier_no_fence();  // block e landed for every wave; the buffer of block e - 1 is free
    if (e + LS::NBUF - 1 < L) issue(blk(e + LS::NBUF - 1), (e + LS::NBUF - 1) % LS::NBUF);
    const unsigned char* pkb = smem + (e % LS::NBUF) * LS::STAGE;
    const unsigned char* pvb = pkb + LS::TILE;
#pragma unroll
    for (int s2 = 0; s2 < TPW; ++s2) {
      const int t = wave + 4 * s2;
      if (t < NTILE) {
        const int ra = t / DT, rc = t % DT;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rowa = 32 * ra + l32, rowb = 32 * rc + l32;
          const bf16x8 av = lds_read16(pkb + rowa * T::VROWB + T::vchunk(rowa, 2 * g + h2) * 16);
          const bf16x8 bv = lds_read16(pvb + rowb * T::VROWB + T::vchunk(rowb, 2 * g + h2) * 16);
          acc[s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[s2], 0, 0, 0);
          if (rc == 0) {
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) zp[s2] += (float)av[e2];
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the stage buffers, which Hs overlays
  // the listed route subtracts from the totals: two uniform branches, so that
  // the totals' loads are issued together rather than one wait per element
  const float* Ht = lin_h + (size_t)bh * D * D;
  if (use_kept) {
#pragma unroll
    for (int s2 = 0; s2 < TPW; ++s2) {
      const int t = wave + 4 * s2;
      if (t < NTILE) {
        const int ra = t / DT, rc = t % DT;
        float tot[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tot[r] = Ht[(size_t)(32 * ra + 8 * (r >> 2) + 4 * h2 + (r & 3)) * D + 32 * rc + l32];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          Hs[(32 * ra + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HP + 32 * rc + l32] = tot[r] - acc[s2][r];
      }
    }
  } else {
#pragma unroll
    for (int s2 = 0; s2 < TPW; ++s2) {
      const int t = wave + 4 * s2;
      if (t < NTILE) {
        const int ra = t / DT, rc = t % DT;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          Hs[(32 * ra + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HP + 32 * rc + l32] = acc[s2][r];
      }
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < TPW; ++s2) {
    const int t = wave + 4 * s2;
    if (t < NTILE && t % DT == 0) {
      const float zt = zp[s2] + __shfl_xor(zp[s2], 32);
      const int a = 32 * (t / DT) + l32;
      if (h2 == 0) zs[a] = use_kept ? lin_z[(size_t)bh * D + a] - zt : zt;
    }
  }
  __syncthreads();

}

// ------------------------------------------------- linear-branch totals
// Split-K partials of H_tot = sum_u phi(K_u)^T V_u (d x d, row = phi index)
// and z_tot = sum_u phi(K_u) from the packed tiles: workgroup (split, bh)
// covers blocks j = split, split + kLinSplit, ...; D/32 waves, wave w owns
// rows 32w..32w+31. Operands come straight from the packed global tiles.
template <int D>
__global__ __launch_bounds__(D * 2) void linear_total_kernel(const uint16_t* __restrict__ phikt,
                                                             const uint16_t* __restrict__ vt,
                                                             float* __restrict__ part_h,
                                                             float* __restrict__ part_z,
                                                             int n_k,
                                                             const int32_t* __restrict__ lin_on,
                                                             int H) {
  constexpr int DT = D / 32;
  const int split = blockIdx.x, bh = blockIdx.y;
  if (!lin_on[bh % H]) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  floatx16 hacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) hacc[i][r] = 0.0f;
  float zp = 0.0f;
  const size_t tile = (size_t)D * BK;
  for (int j = split; j < n_k; j += kLinSplit) {
    const uint16_t* pk = phikt + ((size_t)bh * n_k + j) * tile + (size_t)(32 * wave + l32) * BK;
    const uint16_t* vv = vt + ((size_t)bh * n_k + j) * tile + (size_t)l32 * BK;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(pk + 16 * g + 8 * h2);
#pragma unroll
      for (int e = 0; e < 8; ++e) zp += (float)a[e];
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(vv + (size_t)32 * i * BK + 16 * g + 8 * h2);
        hacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, hacc[i], 0, 0, 0);
      }
    }
  }
  float* ph = part_h + ((size_t)bh * kLinSplit + split) * D * D;
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int a = 32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3);
      ph[(size_t)a * D + 32 * i + l32] = hacc[i][r];
    }
  zp += __shfl_xor(zp, 32);
  if (h2 == 0) part_z[((size_t)bh * kLinSplit + split) * D + 32 * wave + l32] = zp;
}

// H_tot, z_tot = sums of the kLinSplit partials, in split order. Grid (b*h,
// chunks of 256 entries of H then z); each thread sums one entry, its
// partials loaded eight at a time.
template <int D>
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ part_h,
                                                            const float* __restrict__ part_z,
                                                            float* __restrict__ lin_h,
                                                            float* __restrict__ lin_z,
                                                            const int32_t* __restrict__ lin_on,
                                                            int H) {
  const int bh = blockIdx.x, e = blockIdx.y * 256 + threadIdx.x;
  if (!lin_on[bh % H] || e >= D * D + D) return;
  const bool hpart = e < D * D;
  const float* src = hpart ? part_h + (size_t)bh * kLinSplit * D * D + e
                           : part_z + (size_t)bh * kLinSplit * D + (e - D * D);
  const size_t stride = hpart ? (size_t)D * D : (size_t)D;
  static_assert(kLinSplit % 8 == 0, "whole groups of partials");
  float acc = 0.0f;
  for (int sp = 0; sp < kLinSplit; sp += 8) {
    float v[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = src[(size_t)(sp + x) * stride];
#pragma unroll
    for (int x = 0; x < 8; ++x) acc += v[x];
  }
  if (hpart)
    lin_h[(size_t)bh * D * D + e] = acc;
  else
    lin_z[(size_t)bh * D + (e - D * D)] = acc;
}

// lin_on[h] = 1 unless every weight that head h's linear branch is multiplied
// by (alpha[h]; 1 - alpha[h][c] in the mix, float32) has magnitude <= the
// threshold: post-tuning branch dropping (SALAD page). A NaN weight keeps it.
// Then the (batch, head) pairs b*H + h in increasing order, split by the flag:
// lists[0] = #on, lists[1] = #off, lists[2 ..] those on, lists[2 + B*H ..]
// those off. One workgroup; wave w decides heads w, w + 16, ...
constexpr int kFlagThreads = 1024;
__global__ __launch_bounds__(kFlagThreads) void linear_flags_kernel(
    const float* __restrict__ alpha, int mode, int D, float drop_below, int B, int H,
    int32_t* __restrict__ lin_on, int32_t* __restrict__ lists) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int h = wave; h < H; h += kFlagThreads / 64) {
    bool keep = false;
    if (mode == kLinAdd) {
      keep = lane == 0 && !(fabsf(alpha[h]) <= drop_below);
    } else {
      for (int c = lane; c < D; c += 64)
        keep = keep || !(fabsf(1.0f - alpha[(size_t)h * D + c]) <= drop_below);
    }
    keep = __any(keep);
    if (lane == 0) lin_on[h] = keep ? 1 : 0;
  }
  __syncthreads();
  if (wave != 0) return;
  const int BH = B * H;
  int n_on = 0, n_off = 0;
  for (int base = 0; base < BH; base += 64) {
    const int bh = base + lane;
    const bool valid = bh < BH;
    const bool on = valid && lin_on[bh % H] != 0, off = valid && !on;
    const uint64_t m_on = __ballot(on), m_off = __ballot(off);
    const uint64_t below = (uint64_t(1) << lane) - 1;
    if (on) lists[2 + n_on + __popcll(m_on & below)] = bh;
    if (off) lists[2 + BH + n_off + __popcll(m_off & below)] = bh;
    n_on += __popcll(m_on);
    n_off += __popcll(m_off);
  }
  if (lane == 0) {
    lists[0] = n_on;
    lists[1] = n_off;
  }
}

}  // namespace
}  // namespace sparge
