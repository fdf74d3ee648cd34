// Linear-branch code of the forward and the backward translation units: the
// per-head branch flags (post-tuning branch dropping), the per-key-block
// summaries [H_j, z_j] formed with the V packing, the drop bits, and the
// matrix product over blocks that sums, for every row of the bits, the
// summaries of the blocks it drops. The forward forms H_D, z_D of each query
// block with it; the backward sums the query blocks' dH_D, dz_D per key block
// with the transposed bits.
#pragma once

#include "internal.h"
#include "tiles.h"

namespace sparge {
namespace {

// ------------------------------------------------ linear branch: H_D, z_D
// For every query block i, H_D = sum over the key blocks j it does not list
// of phi(K_j)^T V_j and z_D = sum of phi(K_j) over the same blocks, as a
// matrix product over the key blocks: the per-block summaries H_j, z_j are
// formed once, with the V packing (linear_pack_kernel), the drop matrix
// M[i][j] in {0, 1} once per mask (linear_mdrop_kernel), and [H_D, z_D]_i =
// sum_j M[i][j] [H_j, z_j] on the matrix cores (linear_hd_kernel). The
// forward's attention kernel then forms O_l = phi(Q) H_D / (phi(Q) . z_D) in
// its epilogue. The backward runs the same product a second time, over the
// query blocks with the transposed bits (linear_mtrans_kernel), to sum each
// key block's share of the query blocks' dH_D, dz_D.
//
// Summary rows: hj[bh][j][plane][D*D + D], two bf16 planes (hi = bf16(x),
// lo = bf16(x - hi), about 16 significant bits) of H_j^T (row b = V channel,
// column a = phi channel, at b*D + a), then of z_j (at D*D + a).
template <int D>
constexpr int lin_cols() { return D * D + D; }

// V packing fused with the summaries: one workgroup per (key block j, b h),
// 2*D threads (D / 32 waves). Every thread packs its piece of V_j into vt as
// pack_kernel does; for the heads whose linear branch is evaluated (lin_on)
// it also leaves that piece, and the same piece of bf16(phi(K_j)), in two LDS
// tiles [D][64 slots] (rows of 128 bytes, chunks swizzled as in V^T tiles).
// Wave w then forms rows 32 w .. 32 w + 31 of H_j^T = V_j^T phi(K_j) (the
// 64-slot reduction pairs V and phi(K) slot by slot; keys past N are zero in
// both) with fp32 accumulation of exact bf16 products, D / 32 output tiles
// with phi(K) as the row operand so that each lane holds 4 consecutive
// columns, and writes each plane of its 32-row band, which is contiguous in
// hj, through an LDS staging area as 1 KB store instructions. Threads t < D
// sum phi(K)^T row t over the slots in slot order for z_j.
template <int D>
__global__ __launch_bounds__(2 * D) void linear_pack_kernel(const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ k,
                                                            uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ hj, int N,
                                                            int n_k,
                                                            const int32_t* __restrict__ lin_on,
                                                            int H) {
  constexpr int DT = D / 32, COLS = lin_cols<D>(), ROWB = BK * 2, TBYTES = D * ROWB;
  constexpr int PITCH = D * 2 + 16;  // staging row pitch: 8-byte writes by 32 rows spread out
  constexpr int SMEM = (2 * TBYTES > DT * 32 * PITCH) ? 2 * TBYTES : DT * 32 * PITCH;
  __shared__ __align__(16) unsigned char smem[SMEM];
  unsigned char* const vtile = smem;
  unsigned char* const ptile = smem + TBYTES;
  using T = Tile<D>;
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int q = t & 15, c = t >> 4;
  const int slot0 = 16 * (q >> 2) + 8 * (q & 1) + 4 * ((q >> 1) & 1);
  const bool lin = lin_on[bh % H] != 0;  // the same for the whole workgroup
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (w == 1 && !lin) return;
    const uint16_t* src = (w == 0 ? v : k) + ((size_t)bh * N + (size_t)j * BK) * D + c * 8;
    uint32_t x[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 4 * q + r;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (j * BK + key < N) {
        u = *reinterpret_cast<const uint4*>(src + (size_t)key * D);
        if (w == 1) {  // phi(K), rounded to bf16
          uint32_t* p = &u.x;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p[e] = f32_to_bf16_rne(elu1(bf16_lo(p[e]))) |
                   (f32_to_bf16_rne(elu1(bf16_hi(p[e]))) << 16);
        }
      }
      x[r][0] = u.x; x[r][1] = u.y; x[r][2] = u.z; x[r][3] = u.w;
    }
    uint16_t* dst = vt + ((size_t)bh * n_k + j) * (size_t)D * BK + (size_t)(8 * c) * BK + slot0;
    unsigned char* tl = w == 0 ? vtile : ptile;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // d = 8c + 2e (low halves) and 8c + 2e + 1 (high)
      uint2 lo, hi;
      lo.x = (x[0][e] & 0xFFFFu) | (x[1][e] << 16);
      lo.y = (x[2][e] & 0xFFFFu) | (x[3][e] << 16);
      hi.x = (x[0][e] >> 16) | (x[1][e] & 0xFFFF0000u);
      hi.y = (x[2][e] >> 16) | (x[3][e] & 0xFFFF0000u);
      if (w == 0) {
        *reinterpret_cast<uint2*>(dst + (size_t)(2 * e) * BK) = lo;
        *reinterpret_cast<uint2*>(dst + (size_t)(2 * e + 1) * BK) = hi;
      }
      if (lin) {
        const int r0 = 8 * c + 2 * e, r1 = r0 + 1;
        *reinterpret_cast<uint2*>(tl + r0 * ROWB + (T::vchunk(r0, slot0 >> 3) << 4) + 2 * (slot0 & 7)) = lo;
        *reinterpret_cast<uint2*>(tl + r1 * ROWB + (T::vchunk(r1, slot0 >> 3) << 4) + 2 * (slot0 & 7)) = hi;
      }
    }
  }
  __syncthreads();  // both tiles complete (only heads with lin get here)
  const int lane = t & 63, wave = t >> 6, h2 = lane >> 5, l32 = lane & 31;
  floatx16 acc[DT];
#pragma unroll
  for (int ta = 0; ta < DT; ++ta) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ta][r] = 0.0f;
    const int ra = 32 * ta + l32, rb = 32 * wave + l32;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 pa = lds_read16(ptile + ra * ROWB + (T::vchunk(ra, 2 * ks + h2) << 4));
      const bf16x8 vb = lds_read16(vtile + rb * ROWB + (T::vchunk(rb, 2 * ks + h2) << 4));
      acc[ta] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, acc[ta], 0, 0, 0);
    }
  }
  float z = 0.0f;
  if (t < D) {
#pragma unroll
    for (int ch = 0; ch < BK / 8; ++ch) {
      const bf16x8 p8 = lds_read16(ptile + t * ROWB + (T::vchunk(t, ch) << 4));
#pragma unroll
      for (int e = 0; e < 8; ++e) z += (float)p8[e];
    }
  }
  __syncthreads();  // every wave is done with the tiles before the staging reuses them
  // lane: H^T[b = 32 wave + l32][a = 32 ta + 8 g + 4 h2 + (0..3)] = acc[ta][4 g .. 4 g + 3]
  unsigned char* stg = smem + wave * 32 * PITCH;
  uint16_t* out = hj + ((size_t)bh * n_k + j) * 2 * COLS + (size_t)(32 * wave) * D;
#pragma unroll
  for (int pl = 0; pl < 2; ++pl) {
#pragma unroll
    for (int ta = 0; ta < DT; ++ta)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t w2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = acc[ta][4 * g + 2 * e], x1 = acc[ta][4 * g + 2 * e + 1];
          const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
          w2[e] = pl == 0 ? (h0 | (h1 << 16))
                          : (f32_to_bf16_rne(x0 - __uint_as_float(h0 << 16)) |
                             (f32_to_bf16_rne(x1 - __uint_as_float(h1 << 16)) << 16));
        }
        *reinterpret_cast<uint2*>(stg + l32 * PITCH + 2 * (32 * ta + 8 * g + 4 * h2)) =
            make_uint2(w2[0], w2[1]);
      }
    wave_lds_fence();
#pragma unroll
    for (int it = 0; it < D / 16; ++it) {  // 32 rows x D / 8 chunks, 64 per instruction
      const int idx = 64 * it + lane, row = idx / (D / 8), ch = idx % (D / 8);
      *reinterpret_cast<bf16x8*>(out + (size_t)pl * COLS + row * D + 8 * ch) =
          lds_read16(stg + row * PITCH + 16 * ch);
    }
    wave_lds_fence();
  }
  if (t < D) {
    uint16_t* zo = hj + ((size_t)bh * n_k + j) * 2 * COLS + D * D + t;
    const uint32_t hi = f32_to_bf16_rne(z);
    zo[0] = (uint16_t)hi;
    zo[COLS] = (uint16_t)f32_to_bf16_rne(z - __uint_as_float(hi << 16));
  }
}

// mbits[bh][i][w]: bit b of word w is set where query block i does not list
// key block j = 32 w + b (j < n_k); words of n_kw = ceil(n_k / 32) per row.
// One wave per (b, h, query block): the list as a bitmap in LDS (n_k <=
// kLinMaxKeyBlocks), then its complement.
__global__ __launch_bounds__(256) void linear_mdrop_kernel(const int32_t* __restrict__ kv_idx,
                                                           const int32_t* __restrict__ kv_cnt,
                                                           uint32_t* __restrict__ mbits, int n_k,
                                                           int n_kw, int rows) {
  __shared__ uint32_t bits[4][kLinMaxKeyBlocks / 32];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const int count = min(max(kv_cnt[row], 0), n_k);
  const int32_t* ids = kv_idx + (size_t)row * n_k;
  uint32_t* b = bits[wave];
  for (int w = lane; w < n_kw; w += 64) b[w] = 0u;
  wave_lds_fence();
  for (int e = lane; e < count; e += 64) {
    const int j = min(max(ids[e], 0), n_k - 1);
    atomicOr(&b[j >> 5], 1u << (j & 31));
  }
  wave_lds_fence();
  for (int w = lane; w < n_kw; w += 64) {
    const int left = n_k - 32 * w;  // valid key blocks in this word
    const uint32_t valid = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
    mbits[(size_t)row * n_kw + w] = ~b[w] & valid;
  }
}

// 8 drop flags (bits 0..7 of `byte`) as the bf16 values 0 / 1 of an MFMA
// operand: element e of the result is bit e. `spread` has bit e at e and at
// e + 15, so (spread >> 2t) & 0x10001 has bit 2t at 0 and bit 2t+1 at 16.
__device__ __forceinline__ bf16x8 drop_flags_bf16(uint32_t byte) {
  const uint32_t spread = byte | (byte << 15);
  uint32_t w[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = ((spread >> (2 * t)) & 0x10001u) * 0x3F80u;
  bf16x8 r;
  __builtin_memcpy(&r, w, 16);
  return r;
}

// [H_D, z_D]^T[col][i] = sum_j (hi_j + lo_j)[col] M[i][j]. Workgroup (128
// columns, 256 query blocks, b h), 4 waves of 32 columns x 256 query blocks
// (8 accumulator tiles). The key blocks go 32 at a time in stages of the two
// planes' rows j .. j+31 of the workgroup's columns (16 KB) and one drop-bit
// word per query block (1 KB), in a ring of 4 stage buffers filled three
// stages ahead by direct-to-LDS copies, so that enough bytes are in flight to
// cover the memory latency (rows past n_k repeat the last one; their bits are
// 0). The plane operand (8 consecutive key blocks of one column per lane)
// comes from transposing LDS reads, whose 4 rows x 32 bytes per 16 lanes the
// chunk swizzle c ^ 4 (row mod 4) spreads over all banks; M's operand is
// expanded from the drop bits in registers.
// Output per query block: H_D^T as two bf16 planes [2][D][D] (the same
// hi / lo split), written through LDS as whole 256-byte row pieces, and z_D
// as float32 [D] (the last column tile); heads whose branch is dropped are
// skipped.
template <int D>
__global__ __launch_bounds__(256, 2) void linear_hd_kernel(const uint16_t* __restrict__ hj,
                                                           const uint32_t* __restrict__ mbits,
                                                           uint16_t* __restrict__ hd,
                                                           float* __restrict__ zd, int n_q,
                                                           int n_k, int n_kw,
                                                           const int32_t* __restrict__ lin_on,
                                                           int H) {
  constexpr int COLS = lin_cols<D>(), CB = 128, IB = 256, JB = 32, NS = 4;
  constexpr int HBYTES = 2 * JB * CB * 2, STAGE = HBYTES + IB * 4;
  constexpr int SP = CB * 2 + 16;  // output staging row pitch
  static_assert(2 * 2 * 32 * SP <= NS * STAGE, "two output staging buffers fit the ring");
  __shared__ __align__(16) unsigned char smem[NS * STAGE];
  const int bh = blockIdx.z;
  if (!lin_on[bh % H]) return;
  const int c0 = blockIdx.x * CB, i0 = blockIdx.y * IB;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const uint16_t* hsrc = hj + (size_t)bh * n_k * 2 * COLS;
  const uint32_t* msrc = mbits + ((size_t)bh * n_q + min(i0 + t, n_q - 1)) * n_kw;
  // copies of one stage, 5 per wave: 16 KB of plane rows (copy u: plane u / 2,
  // rows 4 (4 (u % 2) + w) .. +3), then the drop word of query block i0 + t
  auto issue = [&](int st) {
    unsigned char* buf = smem + (st % NS) * STAGE;
    const int jb = st * JB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // lane: row r0 + lane / 16, physical chunk lane % 16
      const int pl = u >> 1, r0 = 4 * (4 * (u & 1) + wave), r = r0 + (lane >> 4);
      const int lc = (lane & 15) ^ ((r & 3) << 2);  // the logical chunk this slot holds
      const int col = min(c0 + 8 * lc, COLS - 8);
      const int jr = min(jb + r, n_k - 1);
      dma16(hsrc + ((size_t)jr * 2 + pl) * COLS + col, buf + pl * (JB * CB * 2) + r0 * (CB * 2));
    }
    dma4(msrc + st, buf + HBYTES + 256 * wave);
  };
  floatx16 acc[IB / 32];
#pragma unroll
  for (int ti = 0; ti < IB / 32; ++ti)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ti][r] = 0.0f;
  // transposing-read addresses (bytes within a plane) for k-step ks and read
  // tt: the lane addresses row 16 ks + 8 h2 + 4 tt + (lane & 15) / 4 and the
  // 4 columns 32 wave + 16 ((lane >> 4) & 1) + 4 (lane & 3)
  const int g16 = lane & 15, colb = 32 * wave + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
  auto tr_addr = [&](int ks, int tt) {
    const int r = 16 * ks + 8 * h2 + 4 * tt + (g16 >> 2);
    const int lc = colb >> 3, pc = lc ^ ((r & 3) << 2);
    return (uint32_t)(r * (CB * 2) + 16 * pc + 2 * (colb & 7));
  };
  const int nb = n_kw;  // stages of 32 key blocks
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nb) issue(st);
  for (int bi = 0; bi < nb; ++bi) {
    // this wave's copies of stage bi landed (the later stages already issued,
    // at most NS - 2 of 5 copies each, may still be in flight) and its LDS
    // reads of stage bi - 1 are done
    const int later = min(nb - 1 - bi, NS - 2);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(0x007A);       // vmcnt(10) lgkmcnt(0)
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0075);  // vmcnt(5) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
    // every wave's copies landed; the buffer of stage bi - 1 is free (a fenced
    // barrier would wait for the later stages' copies too)
    barrier_no_fence();
    if (bi + NS - 1 < nb) issue(bi + NS - 1);
    const unsigned char* buf = smem + (bi % NS) * STAGE;
    const uint32_t pbase = lds_addr(buf);
    static_assert(JB == 32, "two k-steps per stage: eight transposing reads");
    uint32_t ad[8];
    v4i16 fr[8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          ad[4 * ks + 2 * pl + tt] = pbase + pl * (JB * CB * 2) + tr_addr(ks, tt);
    lds_read_tr<8>(fr, ad);
    uint32_t mw[IB / 32];  // drop bits of query block i0 + 32 ti + l32 for this stage
#pragma unroll
    for (int ti = 0; ti < IB / 32; ++ti)
      mw[ti] = *reinterpret_cast<const uint32_t*>(buf + HBYTES + 4 * (32 * ti + l32));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 ahi = join_tr(fr[4 * ks], fr[4 * ks + 1]);
      const bf16x8 alo = join_tr(fr[4 * ks + 2], fr[4 * ks + 3]);
#pragma unroll
      for (int ti = 0; ti < IB / 32; ++ti) {
        const bf16x8 bm = drop_flags_bf16((mw[ti] >> (8 * (2 * ks + h2))) & 0xFFu);
        acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bm, acc[ti], 0, 0, 0);
        acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bm, acc[ti], 0, 0, 0);
      }
    }
  }
  // lane: query block i0 + 32 ti + l32, columns c0 + 32 wave + 8 (r / 4) + 4 h2 + r % 4
  if (c0 >= D * D) {  // the z_D tile: float32, straight from the accumulators
#pragma unroll
    for (int ti = 0; ti < IB / 32; ++ti) {
      const int i = i0 + 32 * ti + l32;
      if (i >= n_q) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = c0 + 32 * wave + 8 * g + 4 * h2;
        if (col < COLS)
          *reinterpret_cast<float4*>(zd + ((size_t)bh * n_q + i) * D + (col - D * D)) =
              make_float4(acc[ti][4 * g], acc[ti][4 * g + 1], acc[ti][4 * g + 2], acc[ti][4 * g + 3]);
      }
    }
    return;
  }
  __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
  for (int ti = 0; ti < IB / 32; ++ti) {
    // both planes of 32 query blocks x the workgroup's 128 columns, rows of SP bytes
    unsigned char* stg = smem + (ti & 1) * (2 * 32 * SP);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x0 = acc[ti][4 * g + 2 * e], x1 = acc[ti][4 * g + 2 * e + 1];
        const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
        hw[e] = h0 | (h1 << 16);
        lw[e] = f32_to_bf16_rne(x0 - __uint_as_float(h0 << 16)) |
                (f32_to_bf16_rne(x1 - __uint_as_float(h1 << 16)) << 16);
      }
      const int ofs = l32 * SP + 2 * (32 * wave + 8 * g + 4 * h2);
      *reinterpret_cast<uint2*>(stg + ofs) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2*>(stg + 32 * SP + ofs) = make_uint2(lw[0], lw[1]);
    }
    __syncthreads();  // the staged rows are complete (and the other buffer's readers are done)
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // 2 planes x 32 rows x 16 chunks, 64 chunks per copy
      const int idx = 64 * (4 * u + wave) + lane;
      const int pl = idx >> 9, row = (idx >> 4) & 31, ch = idx & 15;
      const int i = i0 + 32 * ti + row;
      if (i < n_q)
        *reinterpret_cast<bf16x8*>(hd + (((size_t)bh * n_q + i) * 2 + pl) * D * D + c0 + 8 * ch) =
            lds_read16(stg + pl * 32 * SP + row * SP + 16 * ch);
    }
  }
}

// mtbits[bh][j][w]: bit b of word w is set where query block i = 32 w + b
// (i < n_q) does not list key block j: the transpose of mbits, words of n_qw =
// ceil(n_q / 32) per key block. One thread per word.
__global__ __launch_bounds__(256) void linear_mtrans_kernel(const uint32_t* __restrict__ mbits,
                                                            uint32_t* __restrict__ mtbits,
                                                            int n_q, int n_k, int n_kw, int n_qw,
                                                            int BH) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)BH * n_k * n_qw) return;
  const int w = (int)(e % n_qw), j = (int)((e / n_qw) % n_k), bh = (int)(e / ((size_t)n_qw * n_k));
  const uint32_t* src = mbits + ((size_t)bh * n_q + 32 * w) * n_kw + (j >> 5);
  uint32_t word = 0u;
  for (int b = 0; b < 32 && 32 * w + b < n_q; ++b)
    word |= ((src[(size_t)b * n_kw] >> (j & 31)) & 1u) << b;
  mtbits[e] = word;
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
