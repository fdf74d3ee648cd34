// Linear-branch kernels shared by the forward and the backward translation
// units: the per-head branch flags (post-tuning branch dropping) and the
// totals H_tot = sum_u phi(K_u)^T V_u, z_tot = sum_u phi(K_u).
#pragma once

#include "internal.h"
#include "tiles.h"

namespace sparge {
namespace {

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

// H_tot, z_tot = sums of the kLinSplit partials, in split order.
template <int D>
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ part_h,
                                                            const float* __restrict__ part_z,
                                                            float* __restrict__ lin_h,
                                                            float* __restrict__ lin_z,
                                                            const int32_t* __restrict__ lin_on,
                                                            int H) {
  const int bh = blockIdx.x;
  if (!lin_on[bh % H]) return;
  for (int e = threadIdx.x; e < D * D + D; e += 256) {
    float acc = 0.0f;
    if (e < D * D) {
      for (int sp = 0; sp < kLinSplit; ++sp) acc += part_h[((size_t)bh * kLinSplit + sp) * D * D + e];
      lin_h[(size_t)bh * D * D + e] = acc;
    } else {
      const int a = e - D * D;
      for (int sp = 0; sp < kLinSplit; ++sp) acc += part_z[((size_t)bh * kLinSplit + sp) * D + a];
      lin_z[(size_t)bh * D + a] = acc;
    }
  }
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
