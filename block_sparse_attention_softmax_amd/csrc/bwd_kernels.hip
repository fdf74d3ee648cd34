// Backward of the block-sparse attention (the sparse attention of the
// SpargeAttention2 page is fine-tuned by distillation, section 2B, so its
// gradients are needed). With P = softmax over the kept keys of scale Q K^T,
// O = P V and an upstream gradient dO:
//
//   D_t = dO_t . O_t,  dP = dO V^T,  dS = P * (dP - D),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
//
// where P is recomputed from the forward's per-row log-sum-exp. Two kernels,
// both deterministic (no atomics on the results):
//
//  * dK, dV: one workgroup per (b, h, key block j). It walks the query blocks
//    that list j (the transposed lists built below) in increasing order and
//    accumulates dV^T = dO^T P and dK^T = Q^T dS in registers. S = Q K_j^T is
//    computed with one key per lane (lane % 32) so that P and dS, converted
//    to bf16, feed the second products as B operands unchanged, against
//    dO^T and Q^T taken from the staged Q and dO rows by transposing reads.
//    d = 64 uses 4 waves; d = 128 uses 8 (two per SIMD), with V staged in
//    LDS so that a wave's registers hold only its K row beside the
//    accumulators.
//  * dQ: one workgroup per (b, h, query block), the forward's loop over the
//    row's list: S^T = K Q^T and dP^T = V dO^T with one query per lane, then
//    dQ^T += K^T dS^T against K^T packed like V^T.
//
// Every product takes 16-bit operands with fp32 accumulation: bf16, except
// dQ^T = K^T dS^T, which takes fp16. A row's dS sums to zero, so dQ_t =
// scale sum_u dS_tu (K_u - c) for any c: when the kept keys share a large
// common part (neighbouring tokens of a smooth field) the sum cancels, and
// bf16's 8-bit rounding of dS would break the cancellation; fp16 keeps 11
// bits at the same MFMA rate (dS is small, and K converts to fp16 exactly
// in the range of attention inputs).
#include <algorithm>

#include "internal.h"
#include "linear_common.h"
#include "tiles.h"

namespace sparge {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ halfx8 lds_read16_h(const unsigned char* p) {
  return *reinterpret_cast<const halfx8*>(p);
}

__device__ __forceinline__ halfx8 pack_f16x8(const floatx16& x, int base) {
  halfx8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[base + e];
  return r;
}

// ------------------------------------------------------------ row terms
// D[bh][t] = sum_c dO[t][c] O[t][c] (fp32 from the bf16 values) and
// lse2[bh][t] = lse[bh][t] * log2(e), in rows padded to NP = block_q * n_q
// per (b, h) so that whole query blocks can be copied: padding rows get D = 0
// and lse2 = +inf (P = 0). D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ drow,
                                                       float* __restrict__ lse2, int N, int NP,
                                                       size_t rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  constexpr int RPW = 256 / LPR;
  const size_t row = (size_t)blockIdx.x * RPW + threadIdx.x / LPR;  // padded row
  const int part = threadIdx.x % LPR;
  const size_t bh = row / NP;
  const int t = (int)(row % NP);
  const bool live = row < rows && t < N;
  const size_t src = bh * N + t;
  float acc = 0.0f;
  if (live) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + src * D + part * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(dO + src * D + part * 8);
    const uint32_t* pa = &a.x;
    const uint32_t* pb = &b.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(pa[e]), bf16_lo(pb[e]), acc);
      acc = fmaf(bf16_hi(pa[e]), bf16_hi(pb[e]), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    drow[row] = acc;
    lse2[row] = live ? lse[src] * kLog2e : INFINITY;
  }
}

// ----------------------------------------------------- transposed lists
// cmat[bh][j][i] = how many times row block i lists key block j (entries
// clamped to [0, n_k) and counts to [0, n_k] as the forward does). One wave
// per (b, h, query block).
__global__ __launch_bounds__(256) void col_count_kernel(const int32_t* __restrict__ kv_idx,
                                                        const int32_t* __restrict__ kv_cnt,
                                                        int32_t* __restrict__ cmat, int n_q,
                                                        int n_k, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / n_q, i = row % n_q;
  const int count = min(max(kv_cnt[row], 0), n_k);
  for (int e = lane; e < count; e += 64) {
    const int j = min(max(kv_idx[(size_t)row * n_k + e], 0), n_k - 1);
    atomicAdd(&cmat[((size_t)bh * n_k + j) * n_q + i], 1);
  }
}

// colcnt[bh][j] = sum_i cmat[bh][j][i]; one wave per (b, h, key block).
__global__ __launch_bounds__(256) void col_total_kernel(const int32_t* __restrict__ cmat,
                                                        int32_t* __restrict__ colcnt, int n_q,
                                                        int cols) {
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (col >= cols) return;
  int acc = 0;
  for (int i = lane; i < n_q; i += 64) acc += cmat[(size_t)col * n_q + i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) colcnt[col] = acc;
}

// coloff[bh][j] = sum of colcnt[bh][0 .. j-1], j = 0 .. n_k; one workgroup per
// (b, h): each thread scans a contiguous run, then the run totals are scanned
// through LDS.
__global__ __launch_bounds__(256) void col_scan_kernel(const int32_t* __restrict__ colcnt,
                                                       int32_t* __restrict__ coloff, int n_k) {
  __shared__ int part[256];
  const int bh = blockIdx.x, t = threadIdx.x;
  const int per = (n_k + 255) / 256, b0 = min(t * per, n_k), b1 = min(b0 + per, n_k);
  const int32_t* cc = colcnt + (size_t)bh * n_k;
  int run = 0;
  for (int j = b0; j < b1; ++j) run += cc[j];
  part[t] = run;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int u = 0; u < 256; ++u) {
      const int x = part[u];
      part[u] = acc;
      acc += x;
    }
  }
  __syncthreads();
  int32_t* off = coloff + (size_t)bh * (n_k + 1);
  int acc = part[t];
  for (int j = b0; j < b1; ++j) {
    off[j] = acc;
    acc += cc[j];
  }
  if (t == 255) off[n_k] = acc;
}

// collist[bh][coloff[j] ..] = the query blocks listing key block j, in
// increasing order, each repeated as often as it lists j. One wave per column.
__global__ __launch_bounds__(256) void col_list_kernel(const int32_t* __restrict__ cmat,
                                                       const int32_t* __restrict__ coloff,
                                                       int32_t* __restrict__ collist, int n_q,
                                                       int n_k, int cols) {
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (col >= cols) return;
  const int bh = col / n_k, j = col % n_k;
  int32_t* out = collist + (size_t)bh * n_q * n_k + coloff[(size_t)bh * (n_k + 1) + j];
  int pos = 0;
  for (int base = 0; base < n_q; base += 64) {
    const int i = base + lane;
    const int c = i < n_q ? cmat[(size_t)col * n_q + i] : 0;
    int incl = c;  // inclusive prefix over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    for (int r = 0; r < c; ++r) out[pos + incl - c + r] = i;
    pos += __shfl(incl, 63);
  }
}

// --------------------------------------------------------------- dK, dV
// Workgroup (b, h, key block j), 4 waves: wave w holds keys 32*(w & 1) .. +31
// of the block (one per lane % 32) and takes rows (w >> 1) * BQ/2 .. +BQ/2-1
// of every query block that lists j, as BQ/64 sub-tiles of 32 queries; the
// two row halves are summed at the end.
//
// A stage is one listed query block: its Q and dO rows, lse2 and D, copied
// global -> LDS by direct-to-LDS loads into one of two buffers while the
// waves compute on the other (lane i of a wave's copy lands at LDS base +
// 16 i, so each lane reads the global chunk that the swizzle puts there; rows
// past N read row N - 1, and their lse2 = +inf gives P = dS = 0). The S and dP
// products read the rows as they are; the dV and dK products need them
// transposed (8 queries of one channel per lane, in the slot order of the P
// and dS registers), which transposing LDS reads take from the same rows.

// Q / dO rows in LDS, 16-byte chunks XOR-swizzled per row so that both access
// patterns spread over all 64 banks: 16 lanes reading one chunk of 16
// consecutive rows, and 32 lanes reading 64 bytes of 4 consecutive rows (the
// transposing reads). d = 128: the row's low two bits pick the 64-byte group,
// the next two the chunk within it; d = 64 (two rows per bank cycle) uses row
// bits 1 and 2, 3 likewise.
template <int D>
struct RowTile {
  static constexpr int ROWB = D * 2, CPR = D / 8;
  __device__ static constexpr int swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                    : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
  __device__ static constexpr int chunk(int row, int c) { return c ^ swz(row); }
};

template <int D, int BQ>
struct DkdvStage {
  static constexpr int ROWS = BQ * RowTile<D>::ROWB;  // one tensor's rows
  static constexpr int QS = 0, DS = ROWS, LS = 2 * ROWS, DD = 2 * ROWS + BQ * 4;
  static constexpr int BYTES = 2 * ROWS + 2 * BQ * 4;
};

template <int D, int BQ>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void sparse_attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ drow,
    const int32_t* __restrict__ coloff, const int32_t* __restrict__ collist,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int n_q, int n_k, int total,
    float c, float scale, const float* __restrict__ lin_dk, const float* __restrict__ lin_dv) {
  using RT = RowTile<D>;
  using ST = DkdvStage<D, BQ>;
  constexpr int DT = D / 32, KSTEPS = D / 16, NS = BQ / 64;
  constexpr int CU = BQ * RT::CPR / 256;  // 16-byte copies per thread and tensor
  static_assert(BQ * RT::CPR % 256 == 0, "whole copies per thread");
  __shared__ __align__(16) unsigned char smem[2 * ST::BYTES];

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_k, j = tile % n_k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // copy bases are uniform
  const int h2 = lane >> 5, l32 = lane & 31, kw = 32 * (wave & 1), qh = wave >> 1;
  const size_t head = (size_t)bh * N * D;
  const int NP = n_q * BQ;
  const int key = j * BK + kw + l32;

  bf16x8 kf[KSTEPS], vf[KSTEPS];  // this lane's key row (zero past N)
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    kf[s] = bf16x8{};
    vf[s] = bf16x8{};
    if (key < N) {
      kf[s] = *reinterpret_cast<const bf16x8*>(k + head + (size_t)key * D + 16 * s + 8 * h2);
      vf[s] = *reinterpret_cast<const bf16x8*>(v + head + (size_t)key * D + 16 * s + 8 * h2);
    }
  }
  floatx16 dka[DT], dva[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[i][r] = dva[i][r] = 0.0f;

  // per-thread source offsets (elements) of the row copies within a block
  uint32_t src_ofs[CU];
  int src_row[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int p = u * 256 + threadIdx.x, r = p / RT::CPR;
    src_row[u] = r;
    src_ofs[u] = (uint32_t)(r * D + RT::chunk(r, p % RT::CPR) * 8);
  }
  // transposing reads: lane 16g + 4e + m addresses row R0 + 4*h2 + e of the
  // fragment and the 8 bytes at channel 32 ii + 16 (g & 1) + 4 m; with R0 a
  // multiple of 8 the swizzled chunk is (4 ii + ((R0 >> 2) & 3)) ^ tr_lane
  const int e_l = (lane >> 2) & 3, m_l = lane & 3, g1 = (lane >> 4) & 1;
  const int tr_swz = D == 128 ? ((e_l << 2) | h2) : ((((e_l >> 1) & 1) << 2) | h2);
  const int tr_lane = (2 * g1 + (m_l >> 1)) ^ tr_swz;
  const uint32_t tr_row = (uint32_t)((4 * h2 + e_l) * RT::ROWB + 8 * (m_l & 1));

  const int beg = coloff[(size_t)bh * (n_k + 1) + j], end = coloff[(size_t)bh * (n_k + 1) + j + 1];
  const int32_t* lst = collist + (size_t)bh * n_q * n_k;
  auto issue = [&](int r0, unsigned char* buf) {  // the rows of query block r0 / BQ
    const uint16_t* qsrc = q + head + (size_t)r0 * D;
    const uint16_t* dsrc = dO + head + (size_t)r0 * D;
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const uint32_t back = (uint32_t)max(r0 + src_row[u] - (N - 1), 0) * D;  // rows past N
      unsigned char* dst = buf + (u * 256 + wave * 64) * 16;
      dma16(qsrc + src_ofs[u] - back, dst + ST::QS);
      dma16(dsrc + src_ofs[u] - back, dst + ST::DS);
    }
    if (wave < 2 * NS) {  // lse2 (waves 0 .. NS-1) and D (the next NS), 64 rows each
      const int part = wave % NS;
      const float* src = (wave < NS ? lse2 : drow) + (size_t)bh * NP + r0 + 64 * part + lane;
      dma4(src, buf + (wave < NS ? ST::LS : ST::DD) + 256 * part);
    }
  };

  if (beg < end) issue(min(max(lst[beg], 0), n_q - 1) * BQ, smem);
  for (int e = beg; e < end; ++e) {
    const int nxt = e + 1 < end ? min(max(lst[e + 1], 0), n_q - 1) : 0;
    unsigned char* const buf = smem + ((e - beg) & 1) * ST::BYTES;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of the stage landed
    __syncthreads();                     // every wave's copies landed, the other buffer is free
    if (e + 1 < end) issue(nxt * BQ, smem + ((e - beg + 1) & 1) * ST::BYTES);
    const uint32_t bufa = lds_addr(buf) + tr_row;

    // S = Q K^T and dP = dO V^T for every sub-tile's 32 queries x the wave's
    // 32 keys first: 2 NS independent accumulator chains
    floatx16 Sa[NS], dPa[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      const int qr = qh * (BQ / 2) + 32 * n + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) Sa[n][r] = dPa[n][r] = 0.0f;
      bf16x8 fa[KSTEPS], fb[KSTEPS];  // every fragment first: one wait, not one per k-step
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int ch = RT::chunk(qr, 2 * s + h2);
        fa[s] = lds_read16(buf + ST::QS + qr * RT::ROWB + ch * 16);
        fb[s] = lds_read16(buf + ST::DS + qr * RT::ROWB + ch * 16);
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        Sa[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s], kf[s], Sa[n], 0, 0, 0);
        dPa[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s], vf[s], dPa[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      const int qb = qh * (BQ / 2) + 32 * n;  // the sub-tile's first row in the block
      floatx16& S = Sa[n];
      floatx16& dP = dPa[n];
      // P = 2^(S c - lse2), dS = P (dP - D); register r holds row
      // qb + 8*(r/4) + 4*h2 + r%4 (the row terms are read as 16-byte
      // fragments: as float4 the compiler waits here for the next stage's
      // copies in flight into the other buffer)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int t0 = qb + 8 * gg + 4 * h2;
        const float4 l4 = __builtin_bit_cast(float4, lds_read16(buf + ST::LS + 4 * t0));
        const float4 d4 = __builtin_bit_cast(float4, lds_read16(buf + ST::DD + 4 * t0));
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int r = 4 * gg + e2;
          const float p = __builtin_amdgcn_exp2f(fmaf(S[r], c, -lv[e2]));
          S[r] = p;
          dP[r] = p * (dP[r] - dv4[e2]);
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS: k-slots 0..3 of half t are rows
      // qb + 16 t + 4 h2 + 0..3, slots 4..7 the same + 8
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pb = pack_bf16x8(S, 8 * t);
        const bf16x8 sb2 = pack_bf16x8(dP, 8 * t);
        const int R0 = qb + 16 * t;
        const int C0 = (R0 >> 2) & 3, C1 = ((R0 + 8) >> 2) & 3;
        // all of the half's fragments in one block of reads, then its products
        uint32_t ad[4 * DT];
        v4i16 fr[4 * DT];
#pragma unroll
        for (int ii = 0; ii < DT; ++ii) {
          const uint32_t o0 = (uint32_t)(R0 * RT::ROWB + (((4 * ii + C0) ^ tr_lane) << 4));
          const uint32_t o1 = (uint32_t)((R0 + 8) * RT::ROWB + (((4 * ii + C1) ^ tr_lane) << 4));
          ad[4 * ii] = bufa + ST::DS + o0;
          ad[4 * ii + 1] = bufa + ST::DS + o1;
          ad[4 * ii + 2] = bufa + ST::QS + o0;
          ad[4 * ii + 3] = bufa + ST::QS + o1;
        }
        lds_read_tr<4 * DT>(fr, ad);
#pragma unroll
        for (int ii = 0; ii < DT; ++ii) {
          dva[ii] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_tr(fr[4 * ii], fr[4 * ii + 1]), pb,
                                                            dva[ii], 0, 0, 0);
          dka[ii] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_tr(fr[4 * ii + 2], fr[4 * ii + 3]),
                                                            sb2, dka[ii], 0, 0, 0);
        }
      }
    }
  }

  // sum the two row halves: waves 2, 3 hand theirs to waves 0, 1
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [2 key halves][2][DT][16][64]
  static_assert(2 * 2 * DT * 16 * 64 * 4 <= 2 * ST::BYTES, "reduction must fit");
  const int kh = wave & 1;
  if (qh == 1) {
#pragma unroll
    for (int ii = 0; ii < DT; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[(((kh * 2 + 0) * DT + ii) * 16 + r) * 64 + lane] = dka[ii][r];
        red[(((kh * 2 + 1) * DT + ii) * 16 + r) * 64 + lane] = dva[ii][r];
      }
  }
  __syncthreads();
  if (qh == 0 && key < N) {
    uint16_t* krow_p = dk + head + (size_t)key * D;
    uint16_t* vrow_p = dv + head + (size_t)key * D;
#pragma unroll
    for (int ii = 0; ii < DT; ++ii)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float yk[4], yv[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int r = 4 * gg + e2;
          yk[e2] = scale * (dka[ii][r] + red[(((kh * 2 + 0) * DT + ii) * 16 + r) * 64 + lane]);
          yv[e2] = dva[ii][r] + red[(((kh * 2 + 1) * DT + ii) * 16 + r) * 64 + lane];
        }
        const int d0 = 32 * ii + 8 * gg + 4 * h2;
        if (lin_dk) {  // the linear branch's share, float32
          const float4 lk = *reinterpret_cast<const float4*>(lin_dk + head + (size_t)key * D + d0);
          const float4 lv = *reinterpret_cast<const float4*>(lin_dv + head + (size_t)key * D + d0);
          yk[0] += lk.x; yk[1] += lk.y; yk[2] += lk.z; yk[3] += lk.w;
          yv[0] += lv.x; yv[1] += lv.y; yv[2] += lv.z; yv[3] += lv.w;
        }
        uint2 pk;
        pk.x = pack2_bf16(yk[0], yk[1]);
        pk.y = pack2_bf16(yk[2], yk[3]);
        *reinterpret_cast<uint2*>(krow_p + d0) = pk;
        pk.x = pack2_bf16(yv[0], yv[1]);
        pk.y = pack2_bf16(yv[2], yv[3]);
        *reinterpret_cast<uint2*>(vrow_p + d0) = pk;
      }
  }
}

// d = 128: 8 waves, two per SIMD. Holding a key row of both K and V in
// registers (64 VGPRs) beside the 128 of the dK, dV accumulators leaves too
// little for two waves per SIMD, so V of the block is staged in LDS once and
// each wave keeps only its K row. Wave w holds keys 32 (w & 1) .. +31 and
// rows 32 (w >> 1) .. +31 of each 128-row stage. A stage is two 64-row
// segments: the halves of one listed query block (block_q = 128) or two
// consecutive listed blocks (block_q = 64); when the list leaves an odd
// segment count, the last stage's second segment is copied but not computed.
// The four row quarters are summed at the end in two rounds through LDS.
template <int BQ>
__global__ __launch_bounds__(512, 1) void sparse_attn_bwd_dkdv8_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ drow,
    const int32_t* __restrict__ coloff, const int32_t* __restrict__ collist,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int n_q, int n_k, int total,
    float c, float scale, const float* __restrict__ lin_dk, const float* __restrict__ lin_dv) {
  constexpr int D = 128, SB = 128, SEG = 64, SPB = BQ / SEG;
  using RT = RowTile<D>;
  using ST = DkdvStage<D, SB>;
  constexpr int DT = D / 32, KSTEPS = D / 16;
  constexpr int CU = SB * RT::CPR / 512;  // 16-byte copies per thread and tensor
  constexpr int VB = BK * RT::ROWB;       // the block's V rows
  static_assert(CU == 4 && BQ % SEG == 0, "copy split");
  __shared__ __align__(16) unsigned char smem[2 * ST::BYTES + VB];
  unsigned char* const vt = smem + 2 * ST::BYTES;

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_k, j = tile % n_k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // copy bases are uniform
  const int h2 = lane >> 5, l32 = lane & 31, kw = 32 * (wave & 1), qq = wave >> 1;
  const size_t head = (size_t)bh * N * D;
  const int NP = n_q * BQ;
  const int key = j * BK + kw + l32;

  bf16x8 kf[KSTEPS];  // this lane's key row (zero past N)
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    kf[s] = bf16x8{};
    if (key < N) kf[s] = *reinterpret_cast<const bf16x8*>(k + head + (size_t)key * D + 16 * s + 8 * h2);
  }
  // V rows of the block, swizzled like the stage rows (rows past N read row N - 1)
#pragma unroll
  for (int u = 0; u < BK * RT::CPR / 512; ++u) {
    const int p = u * 512 + threadIdx.x, r = p / RT::CPR, ch = p % RT::CPR;
    const int row = min(j * BK + r, N - 1);
    *reinterpret_cast<bf16x8*>(vt + r * RT::ROWB + RT::chunk(r, ch) * 16) =
        *reinterpret_cast<const bf16x8*>(v + head + (size_t)row * D + ch * 8);
  }
  floatx16 dka[DT], dva[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[i][r] = dva[i][r] = 0.0f;

  const int e_l = (lane >> 2) & 3, m_l = lane & 3, g1 = (lane >> 4) & 1;
  const int tr_swz = (e_l << 2) | h2;
  const int tr_lane = (2 * g1 + (m_l >> 1)) ^ tr_swz;
  const uint32_t tr_row = (uint32_t)((4 * h2 + e_l) * RT::ROWB + 8 * (m_l & 1));

  const int beg = coloff[(size_t)bh * (n_k + 1) + j], end = coloff[(size_t)bh * (n_k + 1) + j + 1];
  const int32_t* lst = collist + (size_t)bh * n_q * n_k;
  const int nseg = (end - beg) * SPB, stages = (nseg + 1) / 2;
  auto seg_row = [&](int g) {  // first query row of segment g
    return min(max(lst[beg + g / SPB], 0), n_q - 1) * BQ + (g % SPB) * SEG;
  };
  auto issue = [&](int t, unsigned char* buf) {  // the two segments of stage t
    const int ra = seg_row(2 * t), rb = 2 * t + 1 < nseg ? seg_row(2 * t + 1) : ra;
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int p = u * 512 + threadIdx.x, r = p / RT::CPR;  // r / 64 == u / 2
      const int r0 = u < CU / 2 ? ra : rb, rr = r % SEG;
      const uint32_t back = (uint32_t)max(r0 + rr - (N - 1), 0) * D;  // rows past N
      const uint32_t ofs = (uint32_t)(rr * D + RT::chunk(r, p % RT::CPR) * 8);
      unsigned char* dst = buf + (u * 512 + wave * 64) * 16;
      dma16(q + head + (size_t)r0 * D + ofs - back, dst + ST::QS);
      dma16(dO + head + (size_t)r0 * D + ofs - back, dst + ST::DS);
    }
    if (wave < 4) {  // lse2 (waves 0, 1) and D (waves 2, 3), one segment each
      const int sg = wave & 1;
      const float* src = (wave < 2 ? lse2 : drow) + (size_t)bh * NP + (sg ? rb : ra) + lane;
      dma4(src, buf + (wave < 2 ? ST::LS : ST::DD) + 256 * sg);
    }
  };

  if (stages > 0) issue(0, smem);
  for (int t = 0; t < stages; ++t) {
    unsigned char* const buf = smem + (t & 1) * ST::BYTES;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of the stage landed
    __syncthreads();                     // every wave's copies landed, the other buffer is free
    if (t + 1 < stages) issue(t + 1, smem + ((t + 1) & 1) * ST::BYTES);
    if (2 * t + (qq >> 1) >= nseg) continue;  // an uncomputed trailing segment
    const uint32_t bufa = lds_addr(buf) + tr_row;
    const int qb = 32 * qq, qr = qb + l32, vr = kw + l32;

    // S = Q K^T and dP = dO V^T for the wave's 32 rows x 32 keys
    floatx16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int ch = RT::chunk(qr, 2 * s + h2);
      const bf16x8 fa = lds_read16(buf + ST::QS + qr * RT::ROWB + ch * 16);
      const bf16x8 fb = lds_read16(buf + ST::DS + qr * RT::ROWB + ch * 16);
      const bf16x8 vb = lds_read16(vt + vr * RT::ROWB + RT::chunk(vr, 2 * s + h2) * 16);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, kf[s], S, 0, 0, 0);
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, vb, dP, 0, 0, 0);
    }
    // P = 2^(S c - lse2), dS = P (dP - D); register r holds stage row
    // qb + 8*(r/4) + 4*h2 + r%4
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int t0 = qb + 8 * gg + 4 * h2;
      const float4 l4 = __builtin_bit_cast(float4, lds_read16(buf + ST::LS + 4 * t0));
      const float4 d4 = __builtin_bit_cast(float4, lds_read16(buf + ST::DD + 4 * t0));
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int r = 4 * gg + e2;
        const float p = __builtin_amdgcn_exp2f(fmaf(S[r], c, -lv[e2]));
        S[r] = p;
        dP[r] = p * (dP[r] - dv4[e2]);
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS, in two halves of 16 rows; P and dS
    // go to bf16 first (their float32 registers are then free), and the
    // transposed fragments are read two channel groups at a time
    const bf16x8 pb[2] = {pack_bf16x8(S, 0), pack_bf16x8(S, 8)};
    const bf16x8 sb[2] = {pack_bf16x8(dP, 0), pack_bf16x8(dP, 8)};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R0 = qb + 16 * h;
      const int C0 = (R0 >> 2) & 3, C1 = ((R0 + 8) >> 2) & 3;
#pragma unroll
      for (int i2 = 0; i2 < DT; i2 += 2) {
        uint32_t ad[8];
        v4i16 fr[8];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int ii = i2 + x;
          const uint32_t o0 = (uint32_t)(R0 * RT::ROWB + (((4 * ii + C0) ^ tr_lane) << 4));
          const uint32_t o1 = (uint32_t)((R0 + 8) * RT::ROWB + (((4 * ii + C1) ^ tr_lane) << 4));
          ad[4 * x] = bufa + ST::DS + o0;
          ad[4 * x + 1] = bufa + ST::DS + o1;
          ad[4 * x + 2] = bufa + ST::QS + o0;
          ad[4 * x + 3] = bufa + ST::QS + o1;
        }
        lds_read_tr<8>(fr, ad);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int ii = i2 + x;
          dva[ii] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_tr(fr[4 * x], fr[4 * x + 1]),
                                                            pb[h], dva[ii], 0, 0, 0);
          dka[ii] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_tr(fr[4 * x + 2], fr[4 * x + 3]),
                                                            sb[h], dka[ii], 0, 0, 0);
        }
      }
    }
  }

  // sum the four row quarters: quarters 2, 3 into 0, 1, then 1 into 0
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][2][DT][16][64]
  static_assert(4 * 2 * DT * 16 * 64 * 4 <= 2 * ST::BYTES, "reduction must fit");
  const int kh = wave & 1;
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const int hi = round == 0 ? 2 : 1;  // quarters [hi, 2 hi) hand theirs to [0, hi)
    __syncthreads();
    if (qq >= hi && qq < 2 * hi) {
      const int slot = (qq - hi) * 2 + kh;
#pragma unroll
      for (int ii = 0; ii < DT; ++ii)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[(((slot * 2 + 0) * DT + ii) * 16 + r) * 64 + lane] = dka[ii][r];
          red[(((slot * 2 + 1) * DT + ii) * 16 + r) * 64 + lane] = dva[ii][r];
        }
    }
    __syncthreads();
    if (qq < hi) {
      const int slot = qq * 2 + kh;
#pragma unroll
      for (int ii = 0; ii < DT; ++ii)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dka[ii][r] += red[(((slot * 2 + 0) * DT + ii) * 16 + r) * 64 + lane];
          dva[ii][r] += red[(((slot * 2 + 1) * DT + ii) * 16 + r) * 64 + lane];
        }
    }
  }
  if (qq == 0 && key < N) {
    uint16_t* krow_p = dk + head + (size_t)key * D;
    uint16_t* vrow_p = dv + head + (size_t)key * D;
#pragma unroll
    for (int ii = 0; ii < DT; ++ii)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float yk[4], yv[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          yk[e2] = scale * dka[ii][4 * gg + e2];
          yv[e2] = dva[ii][4 * gg + e2];
        }
        const int d0 = 32 * ii + 8 * gg + 4 * h2;
        if (lin_dk) {  // the linear branch's share, float32
          const float4 lk = *reinterpret_cast<const float4*>(lin_dk + head + (size_t)key * D + d0);
          const float4 lv = *reinterpret_cast<const float4*>(lin_dv + head + (size_t)key * D + d0);
          yk[0] += lk.x; yk[1] += lk.y; yk[2] += lk.z; yk[3] += lk.w;
          yv[0] += lv.x; yv[1] += lv.y; yv[2] += lv.z; yv[3] += lv.w;
        }
        uint2 pk;
        pk.x = pack2_bf16(yk[0], yk[1]);
        pk.y = pack2_bf16(yk[2], yk[3]);
        *reinterpret_cast<uint2*>(krow_p + d0) = pk;
        pk.x = pack2_bf16(yv[0], yv[1]);
        pk.y = pack2_bf16(yv[2], yv[3]);
        *reinterpret_cast<uint2*>(vrow_p + d0) = pk;
      }
  }
}

// ------------------------------------------------------------------- dQ
// Workgroup (b, h, query block), BQ/32 waves of 32 queries (one per lane % 32)
// walking the row's list: S^T = K Q^T, dP^T = V dO^T, P^T, dS^T and
// dQ^T += K^T dS^T. K_j and V_j rows are copied global -> LDS by direct-to-LDS
// loads, double-buffered (the copies of block e+1 run during block e); the
// packed fp16 K_j^T tile is single-buffered and refilled once every wave has
// finished its dQ product, so that copy overlaps the next block's S^T and
// dP^T products. 5 tiles: 80 KB for d = 128, two workgroups per CU.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, (D == 128 && BQ == 64) ? 1 : 2) void sparse_attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ kt, const float* __restrict__ lse2,
    const float* __restrict__ drow, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ dq, int N, int n_q, int n_k,
    int total, float c, float scale, const float* __restrict__ lin_dq) {
  using T = Tile<D>;
  constexpr int DT = D / 32, KSTEPS = D / 16, NT = BQ * 2;
  constexpr int KU = 64 * T::KCPR / NT, VU = D * T::VCPR / NT;  // 16-byte copies per thread
  static_assert(64 * T::KCPR % NT == 0 && D * T::VCPR % NT == 0, "whole copies per thread");
  __shared__ __align__(16) unsigned char smem[5 * T::BYTES];
  unsigned char* const kbuf = smem;                // K rows, two buffers
  unsigned char* const vbuf = smem + 2 * T::BYTES;  // V rows, two buffers
  unsigned char* const kts = smem + 4 * T::BYTES;   // K^T, fp16, packed

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // copy bases are uniform
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const int qrow = qi * BQ + wave * 32 + l32;
  const bool valid = qrow < N;

  bf16x8 qf[KSTEPS], df[KSTEPS];
  {
    const size_t ro = head + (size_t)min(qrow, N - 1) * D + 8 * h2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8*>(q + ro + 16 * s);
      df[s] = *reinterpret_cast<const bf16x8*>(dO + ro + 16 * s);
    }
  }
  const int NP = n_q * BQ;
  const float lq = valid ? lse2[(size_t)bh * NP + qrow] : INFINITY;
  const float dq_d = valid ? drow[(size_t)bh * NP + qrow] : 0.0f;
  floatx16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  uint32_t krow_ofs[KU], vrow_ofs[VU];
  int krow[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int p = u * NT + threadIdx.x, r = p / T::KCPR;
    krow[u] = r;
    krow_ofs[u] = (uint32_t)(r * D + T::kchunk(r, p % T::KCPR) * 8);
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = u * NT + threadIdx.x, r = p / T::VCPR;
    vrow_ofs[u] = (uint32_t)(r * BK + T::vchunk(r, p % T::VCPR) * 8);
  }
  const int count = min(max(kv_cnt[tile], 0), n_k);
  const int32_t* ids = kv_idx + (size_t)tile * n_k;
  auto jat = [&](int e) { return min(max(ids[e], 0), n_k - 1); };
  auto issue_kv = [&](int j, int b) {  // rows past N read row N - 1 (their P is 0)
    const int key0 = j * BK;
    const uint16_t* ksrc = k + head + (size_t)key0 * D;
    const uint16_t* vsrc = v + head + (size_t)key0 * D;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t back = (uint32_t)max(key0 + krow[u] - (N - 1), 0) * D;
      const int slot = (u * NT + wave * 64) * 16;
      dma16(ksrc + krow_ofs[u] - back, kbuf + b * T::BYTES + slot);
      dma16(vsrc + krow_ofs[u] - back, vbuf + b * T::BYTES + slot);
    }
  };
  auto issue_kt = [&](int j) {
    const uint16_t* src = kt + ((size_t)bh * n_k + j) * D * BK;
#pragma unroll
    for (int u = 0; u < VU; ++u) dma16(src + vrow_ofs[u], kts + (u * NT + wave * 64) * 16);
  };

  if (count > 0) {
    issue_kv(jat(0), 0);
    issue_kt(jat(0));
  }
  for (int e = 0; e < count; ++e) {
    const int j = jat(e);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies for block e landed
    __syncthreads();                     // every wave's copies landed; buffer (e+1)&1 is free
    if (e + 1 < count) issue_kv(jat(e + 1), (e + 1) & 1);
    const unsigned char* ks = kbuf + (e & 1) * T::BYTES;
    const unsigned char* vs = vbuf + (e & 1) * T::BYTES;

    floatx16 S[2], dP[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[tau][r] = dP[tau][r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int ch = 2 * s + h2;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int kr = 32 * tau + l32;
        const bf16x8 a = lds_read16(ks + kr * T::KROWB + T::kchunk(kr, ch) * 16);
        const bf16x8 b = lds_read16(vs + kr * T::KROWB + T::kchunk(kr, ch) * 16);
        S[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], S[tau], 0, 0, 0);
        dP[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, df[s], dP[tau], 0, 0, 0);
      }
    }
    const int nvalid = N - j * BK;  // keys past N take no part
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * tau + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const float p = kk < nvalid ? __builtin_amdgcn_exp2f(fmaf(S[tau][r], c, -lq)) : 0.0f;
        dP[tau][r] = p * (dP[tau][r] - dq_d);
      }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        const halfx8 b = pack_f16x8(dP[tau], 8 * hk);
        const int ch = 4 * tau + 2 * hk + h2;
#pragma unroll
        for (int ii = 0; ii < DT; ++ii) {
          const int row = 32 * ii + l32;
          const halfx8 a = lds_read16_h(kts + row * T::VROWB + T::vchunk(row, ch) * 16);
          acc[ii] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[ii], 0, 0, 0);
        }
      }
    __syncthreads();  // every wave is done with K^T of block e
    if (e + 1 < count) issue_kt(jat(e + 1));
  }
  // dQ leaves through LDS as whole rows (every buffer is free after the
  // loop's last barrier; each wave uses its own 32 x D slice)
  static_assert(BQ * D * 2 <= (int)sizeof(smem), "the dQ tiles must fit the buffers");
  store_rows_via_lds<D>(smem + wave * 32 * D * 2, dq + head, qi * BQ + wave * 32, N, lane,
                        [&](int ii, int gg) {
                          const int d0 = 32 * ii + 8 * gg + 4 * h2;
                          float y[4];
#pragma unroll
                          for (int e2 = 0; e2 < 4; ++e2) y[e2] = scale * acc[ii][4 * gg + e2];
                          if (lin_dq && valid) {  // the linear branch's share, float32
                            const float4 l = *reinterpret_cast<const float4*>(
                                lin_dq + head + (size_t)qrow * D + d0);
                            y[0] += l.x; y[1] += l.y; y[2] += l.z; y[3] += l.w;
                          }
                          uint2 pk;
                          pk.x = pack2_bf16(y[0], y[1]);
                          pk.y = pack2_bf16(y[2], y[3]);
                          return pk;
                        });
}

// ------------------------------------------------ linear branch backward
// The linear branch O_l,t = phi(Q_t) H_D / (phi(Q_t) . z_D) of a query block
// with dropped keys D, H_D = sum_{u in D} phi(K_u)^T V_u, z_D = sum phi(K_u),
// receives G_t = w (*) dO_t (w = alpha[h], or 1 - alpha[h][c] in the mix):
//   dnum = G / den,  dden = -(G . O_l) / den,  dphi(Q_t) = H_D dnum + z_D dden,
//   dH_D = sum_t phi(Q_t)^T dnum_t,  dz_D = sum_t phi(Q_t) dden_t,
// and each dropped key u gets dphi(K_u) += dH_D V_u + dz_D, dV_u += phi(K_u) dH_D.
// The sparse part's D_t = dO_t . O_s,t equals dO_t . O_t - G_t . O_l,t, so the
// row kernel subtracts G . O_l from D.

// LDS of linear_bwd_rows_kernel: H_D (rows of HP floats, row = phi(K)
// channel), z_D, then 32 rows of phi(Q) and dnum (rows of FP floats) and dden.
template <int D>
struct LinRowsLds {
  static constexpr int HP = D + 4, FP = D + 4, CH = 32;
  static constexpr int HS = 0, ZS = HS + D * HP * 4, FQ = ZS + D * 4, DN = FQ + CH * FP * 4,
                       DDEN = DN + CH * FP * 4, BYTES = DDEN + CH * 4;
};

// Per (b, h, query block of D rows), 4 waves. H_D comes from the two bf16
// planes of H_D^T that the dropped-block product left for the query block
// (summed into float32 and transposed into LDS), z_D from its float32 row.
// Then, 32 rows at a time in float32 on the vector units: O_l, dnum, dden,
// the correction of D, dQ_l = dphi(Q) phi'(Q) and the block's dH_D, dz_D,
// written as two bf16 planes (hi, rounded remainder) of D*D + D columns
// (dH_D row-major, then dz_D) for the product that sums them per key block.
// Rows of phi(Q) and dnum in LDS are padded by 4 floats and the dQ loop takes
// channels part + 8 i, so that the 8 rows or channels a wave reads at once
// fall in different banks. Heads whose branch is off and blocks that dropped
// nothing write zeros.
template <int D>
__global__ __launch_bounds__(256, 1) void linear_bwd_rows_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ hd, const float* __restrict__ zd,
    const int32_t* __restrict__ kv_cnt, const int32_t* __restrict__ lin_on,
    const float* __restrict__ alpha, int mode, float* __restrict__ dql,
    uint16_t* __restrict__ dhp, float* __restrict__ drow, int H, int N, int n_q, int n_k, int NP,
    int total) {
  using LS = LinRowsLds<D>;
  constexpr int HP = LS::HP, FP = LS::FP, CH = LS::CH, COLS = lin_cols<D>();
  constexpr int AT = D / 16, CPT = D / 8;  // dH entries per thread per side; channels per thread
  __shared__ __align__(16) unsigned char smem[LS::BYTES];
  float* const Hs = reinterpret_cast<float*>(smem + LS::HS);
  float* const zs = reinterpret_cast<float*>(smem + LS::ZS);
  float* const fq = reinterpret_cast<float*>(smem + LS::FQ);
  float* const dn = reinterpret_cast<float*>(smem + LS::DN);
  float* const dden_s = reinterpret_cast<float*>(smem + LS::DDEN);

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q, h = bh % H;
  const int th = threadIdx.x;
  const size_t head = (size_t)bh * N * D;
  const int row0 = qi * D;
  const int count = min(max(kv_cnt[tile], 0), n_k);
  const int a0 = (th / 16) * AT, c0 = (th % 16) * AT;
  uint16_t* const dh_out = dhp + ((size_t)bh * n_q + qi) * 2 * COLS;

  if (lin_on[h] == 0 || count >= n_k) {  // no linear gradient from this block
    for (int e = th; e < CH * (D / CH) * D; e += 256) {
      const int row = row0 + e / D;
      if (row < N) dql[head + (size_t)row * D + e % D] = 0.0f;
    }
    for (int e = th; e < 2 * COLS / 8; e += 256)
      reinterpret_cast<uint4*>(dh_out)[e] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }

  // ---- H_D (Hs[a][c] = H_D^T[c][a], both planes summed) and z_D
  {
    const uint16_t* hsrc = hd + ((size_t)bh * n_q + qi) * 2 * D * D;
    for (int e = th; e < D * D / 8; e += 256) {
      const int c = 8 * e / D, a8 = 8 * e % D;
      const uint4 hi = *reinterpret_cast<const uint4*>(hsrc + 8 * e);
      const uint4 lo = *reinterpret_cast<const uint4*>(hsrc + D * D + 8 * e);
      const uint32_t* wh = &hi.x;
      const uint32_t* wl = &lo.x;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        Hs[(a8 + 2 * x) * HP + c] = bf16_lo(wh[x]) + bf16_lo(wl[x]);
        Hs[(a8 + 2 * x + 1) * HP + c] = bf16_hi(wh[x]) + bf16_hi(wl[x]);
      }
    }
    if (th < D) zs[th] = zd[((size_t)bh * n_q + qi) * D + th];
    __syncthreads();
  }

  // ---- rows, 32 at a time
  float dh[AT][AT], dzacc[AT];
#pragma unroll
  for (int i = 0; i < AT; ++i) {
    dzacc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < AT; ++j) dh[i][j] = 0.0f;
  }
  const int t = th >> 3, part = th & 7, cb = part * CPT;
  for (int chk = 0; chk < D / CH; ++chk) {
    const int r0 = row0 + chk * CH;
    for (int p = th; p < CH * D / 8; p += 256) {  // phi(Q) of the chunk, zero past N
      const int tt = p / (D / 8), c8 = (p % (D / 8)) * 8;
      float f[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      if (r0 + tt < N) {
        const uint4 u = *reinterpret_cast<const uint4*>(q + head + (size_t)(r0 + tt) * D + c8);
        const uint32_t* w = &u.x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = elu1(bf16_lo(w[e]));
          f[2 * e + 1] = elu1(bf16_hi(w[e]));
        }
      }
      *reinterpret_cast<float4*>(fq + tt * FP + c8) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(fq + tt * FP + c8 + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
    // num_t = phi(Q_t) H_D for this thread's channels, den_t = phi(Q_t) . z_D
    float num[CPT];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) num[cc] = 0.0f;
    for (int a = 0; a < D; ++a) {
      const float f = fq[t * FP + a];
#pragma unroll
      for (int cc = 0; cc < CPT; cc += 4) {
        const float4 hv = *reinterpret_cast<const float4*>(Hs + a * HP + cb + cc);
        num[cc] = fmaf(f, hv.x, num[cc]);
        num[cc + 1] = fmaf(f, hv.y, num[cc + 1]);
        num[cc + 2] = fmaf(f, hv.z, num[cc + 2]);
        num[cc + 3] = fmaf(f, hv.w, num[cc + 3]);
      }
    }
    float den = 0.0f;
    for (int a = cb; a < cb + CPT; ++a) den = fmaf(fq[t * FP + a], zs[a], den);
    den += __shfl_xor(den, 4);
    den += __shfl_xor(den, 2);
    den += __shfl_xor(den, 1);
    const int row = r0 + t;
    const bool live = row < N;
    float g[CPT];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) g[cc] = 0.0f;
    if (live) {
      const uint16_t* dp = dO + head + (size_t)row * D + cb;
#pragma unroll
      for (int cc = 0; cc < CPT; cc += 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(dp + cc);
        const uint32_t* w = &u.x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[cc + 2 * e] = bf16_lo(w[e]);
          g[cc + 2 * e + 1] = bf16_hi(w[e]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc)
        g[cc] *= mode == kLinAdd ? alpha[h] : 1.0f - alpha[(size_t)h * D + cb + cc];
    }
    const float inv_den = live ? 1.0f / den : 0.0f;
    float corr = 0.0f;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      corr = fmaf(g[cc], num[cc] * inv_den, corr);  // G . O_l
      dn[t * FP + cb + cc] = g[cc] * inv_den;         // dnum
    }
    corr += __shfl_xor(corr, 4);
    corr += __shfl_xor(corr, 2);
    corr += __shfl_xor(corr, 1);
    if (part == 0) {
      dden_s[t] = -corr * inv_den;
      if (live) drow[(size_t)bh * NP + row] -= corr;
    }
    __syncthreads();
    // dQ_l = (H_D dnum + z_D dden) phi'(Q), phi' = 1 where phi > 1, else phi;
    // this thread takes channels part + 8 i
    if (live) {
      const float ddn = dden_s[t];
#pragma unroll 2
      for (int i = 0; i < CPT; ++i) {
        const int a = part + 8 * i;
        float acc2 = zs[a] * ddn;
        for (int cc = 0; cc < D; cc += 4) {
          const float4 hv = *reinterpret_cast<const float4*>(Hs + a * HP + cc);
          const float4 dv4 = *reinterpret_cast<const float4*>(dn + t * FP + cc);
          acc2 = fmaf(hv.x, dv4.x, acc2);
          acc2 = fmaf(hv.y, dv4.y, acc2);
          acc2 = fmaf(hv.z, dv4.z, acc2);
          acc2 = fmaf(hv.w, dv4.w, acc2);
        }
        const float f = fq[t * FP + a];
        dql[head + (size_t)row * D + a] = acc2 * (f > 1.0f ? 1.0f : f);
      }
    }
    // dH_D += phi(Q)^T dnum, dz_D += phi(Q)^T dden over the chunk's rows
    for (int t2 = 0; t2 < CH; ++t2) {
      float fa[AT], dc[AT];
#pragma unroll
      for (int i = 0; i < AT; i += 4) {
        const float4 x = *reinterpret_cast<const float4*>(fq + t2 * FP + a0 + i);
        const float4 y = *reinterpret_cast<const float4*>(dn + t2 * FP + c0 + i);
        fa[i] = x.x; fa[i + 1] = x.y; fa[i + 2] = x.z; fa[i + 3] = x.w;
        dc[i] = y.x; dc[i + 1] = y.y; dc[i + 2] = y.z; dc[i + 3] = y.w;
      }
#pragma unroll
      for (int i = 0; i < AT; ++i)
#pragma unroll
        for (int j = 0; j < AT; ++j) dh[i][j] = fmaf(fa[i], dc[j], dh[i][j]);
      const float dd2 = dden_s[t2];
#pragma unroll
      for (int i = 0; i < AT; ++i) dzacc[i] = fmaf(fa[i], dd2, dzacc[i]);
    }
    __syncthreads();  // the next chunk overwrites fq, dn
  }
  // two bf16 planes: hi = bf16(x), lo = bf16(x - hi)
#pragma unroll
  for (int i = 0; i < AT; ++i)
#pragma unroll
    for (int j = 0; j < AT; j += 2) {
      const uint32_t h0 = f32_to_bf16_rne(dh[i][j]), h1 = f32_to_bf16_rne(dh[i][j + 1]);
      const uint32_t l0 = f32_to_bf16_rne(dh[i][j] - __uint_as_float(h0 << 16));
      const uint32_t l1 = f32_to_bf16_rne(dh[i][j + 1] - __uint_as_float(h1 << 16));
      const size_t col = (size_t)(a0 + i) * D + c0 + j;
      *reinterpret_cast<uint32_t*>(dh_out + col) = h0 | (h1 << 16);
      *reinterpret_cast<uint32_t*>(dh_out + COLS + col) = l0 | (l1 << 16);
    }
  if (th % 16 == 0)
#pragma unroll
    for (int i = 0; i < AT; ++i) {
      const uint32_t hz = f32_to_bf16_rne(dzacc[i]);
      dh_out[D * D + a0 + i] = (uint16_t)hz;
      dh_out[COLS + D * D + a0 + i] = (uint16_t)f32_to_bf16_rne(dzacc[i] - __uint_as_float(hz << 16));
    }
}

// The same on the matrix cores (d = 128, 128-row query blocks). Wave w takes
// rows 32 w .. 32 w + 31, one per lane, channels in the accumulator layout of
// the forward's O^T. H_D^T's two planes are copied into LDS with the chunk
// swizzle of linear_bwd_keys_mfma_kernel (direct row reads and 4-row
// transposing reads both conflict-free).
//   num^T = H_D^T phi(Q)^T: H_D^T rows read directly, phi(Q) split into hi +
//     lo bf16 in registers; three products (lo x lo left out), as the forward.
//   den, G = w (*) dO, corr = G . num / den, dnum = G / den, dden = -corr /
//     den (float32, per lane), D -= corr.
//   dQ_l^T = H_D dnum^T + z_D dden, times phi'(Q): dnum stays in its
//     accumulator registers as the B operand, the k order of each 16-channel
//     step being that of the registers (channels 16 p + 8 (e / 4) + 4 h2 +
//     e % 4 of a 32-channel tile), and H_D's matching 8 rows per lane come from
//     two 4-row transposing reads of H_D^T; three products.
//   dH^T = dnum^T phi(Q) over the block's 128 rows: 64 rows at a time, the two
//     waves holding them write phi(Q) and dnum as bf16 hi / lo planes into the
//     space H_D^T used, and every wave takes 2 x 2 of the 16 output tiles from
//     transposing reads of both (8 rows t of one channel per lane); three
//     products. dz = sum_t phi(Q_t) dden_t by threads t < d from the same
//     planes. dH, dz leave as two bf16 planes as in linear_bwd_rows_kernel.
template <int D>
__global__ __launch_bounds__(256, 2) void linear_bwd_rows_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ hd, const float* __restrict__ zd,
    const int32_t* __restrict__ kv_cnt, const int32_t* __restrict__ lin_on,
    const float* __restrict__ alpha, int mode, float* __restrict__ dql,
    uint16_t* __restrict__ dhp, float* __restrict__ drow, int H, int N, int n_q, int n_k, int NP,
    int total) {
  static_assert(D == 128, "rows of 16 chunks, four 32-row waves");
  constexpr int PL = D * D * 2, ROWB = D * 2, KS = D / 16, DT = D / 32, COLS = lin_cols<D>();
  constexpr int HALF = 64 * ROWB;  // one bf16 plane of 64 rows
  constexpr int ZS = 2 * PL, DDN = ZS + D * 4, BYTES = DDN + D * 4;
  __shared__ __align__(16) unsigned char smem[BYTES];
  float* const zs = reinterpret_cast<float*>(smem + ZS);
  float* const ddn = reinterpret_cast<float*>(smem + DDN);

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q, h = bh % H;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h2 = lane >> 5, l32 = lane & 31, g16 = lane & 15;
  const size_t head = (size_t)bh * N * D;
  const int row0 = qi * D;
  const int count = min(max(kv_cnt[tile], 0), n_k);
  uint16_t* const dh_out = dhp + ((size_t)bh * n_q + qi) * 2 * COLS;

  if (lin_on[h] == 0 || count >= n_k) {  // no linear gradient from this block
    for (int e = t; e < D * D / 4; e += 256) {
      const int row = row0 + e / (D / 4);
      if (row < N)
        *reinterpret_cast<float4*>(dql + head + (size_t)row * D + 4 * (e % (D / 4))) =
            make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    for (int e = t; e < 2 * COLS / 8; e += 256)
      reinterpret_cast<uint4*>(dh_out)[e] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  auto swz = [](int r) { return ((r & 3) << 2) | ((r >> 2) & 3); };
  {  // H_D^T planes: 64 copies of 4 rows, 16 per wave
    const uint16_t* hsrc = hd + ((size_t)bh * n_q + qi) * 2 * D * D;
#pragma unroll
    for (int u = 0; u < 2 * D / 16; ++u) {
      const int ci = 4 * u + wave, pl = ci / (D / 4), r0 = 4 * (ci % (D / 4)), r = r0 + (lane >> 4);
      const int lc = (lane & 15) ^ swz(r);
      dma16(hsrc + (size_t)pl * D * D + (size_t)r * D + 8 * lc, smem + pl * PL + r0 * ROWB);
    }
  }
  if (t < D) zs[t] = zd[((size_t)bh * n_q + qi) * D + t];
  // phi(Q) of this lane's row, channels 16 s + 8 h2 .. +7, as hi + lo (0 past
  // N); formed again from Q where the dH planes are written, so that these
  // registers are free during the dQ products
  const int lrow = 32 * wave + l32, row = row0 + lrow;
  const bool live = row < N;
  auto phi_q = [&](int s2, bf16x8& hi, bf16x8& lo) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (live) u = *reinterpret_cast<const uint4*>(q + head + (size_t)row * D + 16 * s2 + 8 * h2);
    const uint32_t* w = &u.x;
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f0 = live ? elu1(bf16_lo(w[e])) : 0.0f;
      const float f1 = live ? elu1(bf16_hi(w[e])) : 0.0f;
      const uint32_t a0 = f32_to_bf16_rne(f0), a1 = f32_to_bf16_rne(f1);
      hw[e] = a0 | (a1 << 16);
      lw[e] = f32_to_bf16_rne(f0 - __uint_as_float(a0 << 16)) |
              (f32_to_bf16_rne(f1 - __uint_as_float(a1 << 16)) << 16);
    }
    __builtin_memcpy(&hi, hw, 16);
    __builtin_memcpy(&lo, lw, 16);
  };
  bf16x8 qh[KS], ql[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) phi_q(s2, qh[s2], ql[s2]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's plane copies landed
  __syncthreads();                     // and every wave's, and z_D

  // ---- num^T: acc[i][r] = num[row][32 i + 8 (r / 4) + 4 h2 + r % 4]
  floatx16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      const int c = 32 * i + l32;
      const int ofs = c * ROWB + 16 * ((2 * s2 + h2) ^ swz(c));
      const bf16x8 hh = lds_read16(smem + ofs), hl = lds_read16(smem + PL + ofs);
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hh, qh[s2], acc[i], 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hh, ql[s2], acc[i], 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hl, qh[s2], acc[i], 0, 0, 0);
    }
  // ---- den, G, corr; acc becomes dnum
  float den = 0.0f;
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      den = fmaf((float)qh[s2][e] + (float)ql[s2][e], zs[16 * s2 + 8 * h2 + e], den);
  den = pair_sum(den);
  const float inv_den = live ? 1.0f / den : 0.0f;
  float gn = 0.0f;
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = 32 * i + 8 * g + 4 * h2;
      uint2 u = make_uint2(0u, 0u);
      if (live) u = *reinterpret_cast<const uint2*>(dO + head + (size_t)row * D + c0);
      const float dv[4] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gv =
            dv[e] * (mode == kLinAdd ? alpha[h] : 1.0f - alpha[(size_t)h * D + c0 + e]);
        gn = fmaf(gv, acc[i][4 * g + e], gn);
        acc[i][4 * g + e] = gv * inv_den;  // dnum
      }
    }
  const float corr = pair_sum(gn) * inv_den;  // G . O_l
  const float dden = -corr * inv_den;
  if (h2 == 0) {
    ddn[lrow] = dden;
    if (live) drow[(size_t)bh * NP + row] -= corr;
  }
  // ---- dQ_l^T: dq[ta][r] at channel a = 32 ta + 8 (r / 4) + 4 h2 + r % 4
  floatx16 dq[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.0f;
  const uint32_t base = lds_addr(smem);
  const int colq = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 bh_, bl_;  // dnum of channels 32 i + 16 p + 8 (e / 4) + 4 h2 + e % 4
      {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = acc[i][8 * p + 2 * e], x1 = acc[i][8 * p + 2 * e + 1];
          const uint32_t a0 = f32_to_bf16_rne(x0), a1 = f32_to_bf16_rne(x1);
          hw[e] = a0 | (a1 << 16);
          lw[e] = f32_to_bf16_rne(x0 - __uint_as_float(a0 << 16)) |
                  (f32_to_bf16_rne(x1 - __uint_as_float(a1 << 16)) << 16);
        }
        __builtin_memcpy(&bh_, hw, 16);
        __builtin_memcpy(&bl_, lw, 16);
      }
#pragma unroll
      for (int tp = 0; tp < DT / 2; ++tp) {  // two output tiles per batch of 8 reads
        uint32_t ad[8];
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const int r = 32 * i + 16 * p + 8 * tt + 4 * h2 + (g16 >> 2);
              const int colb = 32 * (2 * tp + y) + colq;
              ad[4 * y + 2 * pl + tt] =
                  base + pl * PL + r * ROWB + 16 * ((colb >> 3) ^ swz(r)) + 2 * (colb & 7);
            }
        v4i16 fr[8];
        lds_read_tr<8>(fr, ad);
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int ta = 2 * tp + y;
          const bf16x8 ah = join_tr(fr[4 * y], fr[4 * y + 1]), al = join_tr(fr[4 * y + 2], fr[4 * y + 3]);
          dq[ta] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh_, dq[ta], 0, 0, 0);
          dq[ta] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl_, dq[ta], 0, 0, 0);
          dq[ta] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh_, dq[ta], 0, 0, 0);
        }
      }
    }
  if (live) {
#pragma unroll
    for (int ta = 0; ta < DT; ++ta)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = 32 * ta + 8 * g + 4 * h2;
        const uint2 u = *reinterpret_cast<const uint2*>(q + head + (size_t)row * D + a0);
        const float qv[4] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = elu1(qv[e]);
          y[e] = fmaf(zs[a0 + e], dden, dq[ta][4 * g + e]) * (f > 1.0f ? 1.0f : f);
        }
        *reinterpret_cast<float4*>(dql + head + (size_t)row * D + a0) =
            make_float4(y[0], y[1], y[2], y[3]);
      }
  }
  // ---- dH^T = dnum^T phi(Q) and dz, 64 rows at a time
  __syncthreads();  // every wave is done with H_D^T and has written its dden
  const int ct0 = 2 * (wave >> 1), at0 = 2 * (wave & 1);
  floatx16 dh[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) dh[x][r] = 0.0f;
  float dz = 0.0f;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if ((wave >> 1) == pass) {  // planes: phi(Q) hi, lo, then dnum hi, lo; 64 rows each
      const int lr = 32 * (wave & 1) + l32;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        const int ofs = lr * ROWB + 16 * ((2 * s2 + h2) ^ swz(lr));
        bf16x8 hi, lo;
        phi_q(s2, hi, lo);
        *reinterpret_cast<bf16x8*>(smem + ofs) = hi;
        *reinterpret_cast<bf16x8*>(smem + HALF + ofs) = lo;
      }
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = 32 * i + 8 * g + 4 * h2;
          uint32_t hw[2], lw[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float x0 = acc[i][4 * g + 2 * e], x1 = acc[i][4 * g + 2 * e + 1];
            const uint32_t a0 = f32_to_bf16_rne(x0), a1 = f32_to_bf16_rne(x1);
            hw[e] = a0 | (a1 << 16);
            lw[e] = f32_to_bf16_rne(x0 - __uint_as_float(a0 << 16)) |
                    (f32_to_bf16_rne(x1 - __uint_as_float(a1 << 16)) << 16);
          }
          const int ofs = lr * ROWB + 16 * ((c0 >> 3) ^ swz(lr)) + 2 * (c0 & 7);
          *reinterpret_cast<uint2*>(smem + 2 * HALF + ofs) = make_uint2(hw[0], hw[1]);
          *reinterpret_cast<uint2*>(smem + 3 * HALF + ofs) = make_uint2(lw[0], lw[1]);
        }
    }
    __syncthreads();  // the pass's planes are complete
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // 16 rows per step
      uint32_t ad[8], bd[8];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int r = 16 * ks + 8 * h2 + 4 * tt + (g16 >> 2);
            const int ca = 32 * (ct0 + x) + colq, cb = 32 * (at0 + x) + colq;
            ad[4 * x + 2 * pl + tt] = base + (2 + pl) * HALF + r * ROWB +
                                      16 * ((ca >> 3) ^ swz(r)) + 2 * (ca & 7);
            bd[4 * x + 2 * pl + tt] =
                base + pl * HALF + r * ROWB + 16 * ((cb >> 3) ^ swz(r)) + 2 * (cb & 7);
          }
      v4i16 fa[8], fb[8];
      lds_read_tr<8>(fa, ad);
      lds_read_tr<8>(fb, bd);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const bf16x8 dnh = join_tr(fa[4 * x], fa[4 * x + 1]), dnl = join_tr(fa[4 * x + 2], fa[4 * x + 3]);
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const bf16x8 fqh = join_tr(fb[4 * y], fb[4 * y + 1]), fql = join_tr(fb[4 * y + 2], fb[4 * y + 3]);
          floatx16& d = dh[2 * x + y];
          d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dnh, fqh, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dnh, fql, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dnl, fqh, d, 0, 0, 0);
        }
      }
    }
    if (t < D) {  // dz[a = t] over the pass's rows, in row order
      for (int lr = 0; lr < 64; ++lr) {
        const int ofs = lr * ROWB + 16 * ((t >> 3) ^ swz(lr)) + 2 * (t & 7);
        const float f = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(smem + ofs) << 16) +
                        __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(smem + HALF + ofs) << 16);
        dz = fmaf(f, ddn[64 * pass + lr], dz);
      }
    }
    __syncthreads();  // every wave is done with the pass's planes
  }
  // dH[a][c]: tile (ct0 + x, at0 + y) holds channels c = 32 (ct0 + x) + 8 (r / 4) + 4 h2 + r % 4 of a = 32 (at0 + y) + l32
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx16& d = dh[2 * x + y];
        const int a = 32 * (at0 + y) + l32, c0 = 32 * (ct0 + x) + 8 * g + 4 * h2;
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = d[4 * g + 2 * e], x1 = d[4 * g + 2 * e + 1];
          const uint32_t a0 = f32_to_bf16_rne(x0), a1 = f32_to_bf16_rne(x1);
          hw[e] = a0 | (a1 << 16);
          lw[e] = f32_to_bf16_rne(x0 - __uint_as_float(a0 << 16)) |
                  (f32_to_bf16_rne(x1 - __uint_as_float(a1 << 16)) << 16);
        }
        const size_t col = (size_t)a * D + c0;
        *reinterpret_cast<uint2*>(dh_out + col) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(dh_out + COLS + col) = make_uint2(lw[0], lw[1]);
      }
  if (t < D) {
    const uint32_t hz = f32_to_bf16_rne(dz);
    dh_out[D * D + t] = (uint16_t)hz;
    dh_out[COLS + D * D + t] = (uint16_t)f32_to_bf16_rne(dz - __uint_as_float(hz << 16));
  }
}

// Per (b, h, key block j): G_j = the sum of dH_D over the query blocks that
// dropped j and g_j = that of dz_D, both from the dropped-block product (two
// bf16 planes of G_j, row-major, summed into float32 in LDS; g_j float32),
// then for its 64 keys in float32 dV_l = phi(K) G_j and dK_l = (G_j V + g_j)
// phi'(K). Heads whose branch is off write zeros.
template <int D>
__global__ __launch_bounds__(256, 1) void linear_bwd_keys_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ gp, const float* __restrict__ gz,
    const int32_t* __restrict__ lin_on, float* __restrict__ dkl, float* __restrict__ dvl,
    int H, int N, int n_k, int total) {
  // G row pitch; phi(K) and V row pitch (the 16 keys a wave reads at once
  // fall in different banks); channels per thread
  constexpr int HP = D + 4, KP = D + 4, KPT = D / 4;
  __shared__ __align__(16) float Gs[D * HP];
  __shared__ __align__(16) float gs[D];
  __shared__ __align__(16) float fk[BK * KP];
  __shared__ __align__(16) float vr[BK * KP];
  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_k, j = tile % n_k, h = bh % H;
  const int th = threadIdx.x;
  const size_t head = (size_t)bh * N * D;
  const int key0 = j * BK;
  const int u = th >> 2, cb = (th & 3) * KPT;  // this thread's key and channel quarter
  const bool live = key0 + u < N;

  if (lin_on[h] == 0) {
    if (live)
      for (int cc = 0; cc < KPT; ++cc) {
        dkl[head + (size_t)(key0 + u) * D + cb + cc] = 0.0f;
        dvl[head + (size_t)(key0 + u) * D + cb + cc] = 0.0f;
      }
    return;
  }
  {
    const uint16_t* gsrc = gp + ((size_t)bh * n_k + j) * 2 * D * D;
    for (int e = th; e < D * D / 8; e += 256) {
      const uint4 hi = *reinterpret_cast<const uint4*>(gsrc + 8 * e);
      const uint4 lo = *reinterpret_cast<const uint4*>(gsrc + D * D + 8 * e);
      const uint32_t* wh = &hi.x;
      const uint32_t* wl = &lo.x;
      float g8[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        g8[2 * x] = bf16_lo(wh[x]) + bf16_lo(wl[x]);
        g8[2 * x + 1] = bf16_hi(wh[x]) + bf16_hi(wl[x]);
      }
      float* dst = Gs + (8 * e / D) * HP + 8 * e % D;
      *reinterpret_cast<float4*>(dst) = make_float4(g8[0], g8[1], g8[2], g8[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(g8[4], g8[5], g8[6], g8[7]);
    }
    if (th < D) gs[th] = gz[((size_t)bh * n_k + j) * D + th];
  }
  for (int p = th; p < BK * D / 8; p += 256) {  // phi(K) and V rows of the block, zero past N
    const int uu = p / (D / 8), c8 = (p % (D / 8)) * 8;
    float f[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float w8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (key0 + uu < N) {
      const uint4 kk = *reinterpret_cast<const uint4*>(k + head + (size_t)(key0 + uu) * D + c8);
      const uint4 vv = *reinterpret_cast<const uint4*>(v + head + (size_t)(key0 + uu) * D + c8);
      const uint32_t* wk = &kk.x;
      const uint32_t* wv = &vv.x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = elu1(bf16_lo(wk[e]));
        f[2 * e + 1] = elu1(bf16_hi(wk[e]));
        w8[2 * e] = bf16_lo(wv[e]);
        w8[2 * e + 1] = bf16_hi(wv[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      *reinterpret_cast<float4*>(fk + uu * KP + c8 + e) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
      *reinterpret_cast<float4*>(vr + uu * KP + c8 + e) = make_float4(w8[e], w8[e + 1], w8[e + 2], w8[e + 3]);
    }
  }
  __syncthreads();
  if (!live) return;
  // dV_l[u][c] = sum_a phi(K_u)[a] G[a][c]
  float dvv[KPT];
#pragma unroll
  for (int cc = 0; cc < KPT; ++cc) dvv[cc] = 0.0f;
  for (int a = 0; a < D; ++a) {
    const float f = fk[u * KP + a];
#pragma unroll
    for (int cc = 0; cc < KPT; cc += 4) {
      const float4 gv = *reinterpret_cast<const float4*>(Gs + a * HP + cb + cc);
      dvv[cc] = fmaf(f, gv.x, dvv[cc]);
      dvv[cc + 1] = fmaf(f, gv.y, dvv[cc + 1]);
      dvv[cc + 2] = fmaf(f, gv.z, dvv[cc + 2]);
      dvv[cc + 3] = fmaf(f, gv.w, dvv[cc + 3]);
    }
  }
  float* const vo = dvl + head + (size_t)(key0 + u) * D + cb;
#pragma unroll
  for (int cc = 0; cc < KPT; cc += 4)
    *reinterpret_cast<float4*>(vo + cc) = make_float4(dvv[cc], dvv[cc + 1], dvv[cc + 2], dvv[cc + 3]);
  // dK_l[u][a] = (sum_c G[a][c] V_u[c] + g[a]) phi'(K_u[a]) for the thread's quarter of a
  float* const ko = dkl + head + (size_t)(key0 + u) * D;
  for (int a = cb; a < cb + KPT; ++a) {
    float s2 = gs[a];
    for (int cc = 0; cc < D; cc += 4) {
      const float4 gv = *reinterpret_cast<const float4*>(Gs + a * HP + cc);
      const float4 vv = *reinterpret_cast<const float4*>(vr + u * KP + cc);
      s2 = fmaf(gv.x, vv.x, s2);
      s2 = fmaf(gv.y, vv.y, s2);
      s2 = fmaf(gv.z, vv.z, s2);
      s2 = fmaf(gv.w, vv.w, s2);
    }
    const float f = fk[u * KP + a];
    ko[a] = s2 * (f > 1.0f ? 1.0f : f);
  }
}

// The same on the matrix cores (d = 128). G_j's two planes (row-major
// [a][c]) are copied into LDS with the 16-byte chunk c of row a stored at
// c ^ (4 (a mod 4) + (a / 4) mod 4): 16 consecutive rows read at one chunk,
// and the transposing reads' 4 rows x 32 bytes, both cover all banks. Wave w
// takes keys 32 (w mod 2) .. +31 and channels 64 (w / 2) .. +63:
//   dV_l[u][c] = sum_a phi(K_u)[a] G[a][c]: phi(K) split into two bf16 terms
//     (in registers, from K) against G's planes read transposed (8 rows a of
//     one column c per lane), three products (the lo x lo term left out);
//   dK_l^T[a][u] = sum_c G[a][c] V[u][c], G's planes read directly against V
//     (exact in bf16), two products; then + g[a] and times phi'(K[u][a]).
template <int D>
__global__ __launch_bounds__(256) void linear_bwd_keys_mfma_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ gp, const float* __restrict__ gz,
    const int32_t* __restrict__ lin_on, float* __restrict__ dkl, float* __restrict__ dvl,
    int H, int N, int n_k, int total) {
  static_assert(D == 128, "rows of 16 chunks, two 64-channel halves");
  constexpr int PLANE = D * D * 2, KS = D / 16, ROWB = D * 2;
  __shared__ __align__(16) unsigned char smem[2 * PLANE + D * 4];
  float* const gs = reinterpret_cast<float*>(smem + 2 * PLANE);
  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_k, j = tile % n_k, h = bh % H;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h2 = lane >> 5, l32 = lane & 31, g16 = lane & 15;
  const size_t head = (size_t)bh * N * D;
  const int key0 = j * BK;
  const int ut = wave & 1, chalf = wave >> 1;

  if (lin_on[h] == 0) {
    for (int e = t; e < BK * D / 4; e += 256) {
      const int u = e / (D / 4), c4 = 4 * (e % (D / 4));
      if (key0 + u < N) {
        const size_t o = head + (size_t)(key0 + u) * D + c4;
        *reinterpret_cast<float4*>(dkl + o) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        *reinterpret_cast<float4*>(dvl + o) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    return;
  }
  auto swz = [](int r) { return ((r & 3) << 2) | ((r >> 2) & 3); };
  {  // 64 copies of 4 rows, 16 per wave: lane = row r0 + lane / 16, physical chunk lane % 16
    const uint16_t* gsrc = gp + ((size_t)bh * n_k + j) * 2 * D * D;
#pragma unroll
    for (int u = 0; u < 2 * D / 16; ++u) {
      const int ci = 4 * u + wave, pl = ci / (D / 4), r0 = 4 * (ci % (D / 4)), r = r0 + (lane >> 4);
      const int lc = (lane & 15) ^ swz(r);
      dma16(gsrc + (size_t)pl * D * D + (size_t)r * D + 8 * lc, smem + pl * PLANE + r0 * ROWB);
    }
  }
  if (t < D) gs[t] = gz[((size_t)bh * n_k + j) * D + t];
  // operands of this lane's key (32 ut + l32): phi(K) as hi + lo, V
  const int urow = key0 + 32 * ut + l32;
  const bool ulive = urow < N;
  bf16x8 ph[KS], plo[KS], vb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = kk;
    if (ulive) {
      kk = *reinterpret_cast<const uint4*>(k + head + (size_t)urow * D + 16 * ks + 8 * h2);
      vv = *reinterpret_cast<const uint4*>(v + head + (size_t)urow * D + 16 * ks + 8 * h2);
    }
    const uint32_t* wk = &kk.x;
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f0 = ulive ? elu1(bf16_lo(wk[e])) : 0.0f;
      const float f1 = ulive ? elu1(bf16_hi(wk[e])) : 0.0f;
      const uint32_t a0 = f32_to_bf16_rne(f0), a1 = f32_to_bf16_rne(f1);
      hw[e] = a0 | (a1 << 16);
      lw[e] = f32_to_bf16_rne(f0 - __uint_as_float(a0 << 16)) |
              (f32_to_bf16_rne(f1 - __uint_as_float(a1 << 16)) << 16);
    }
    __builtin_memcpy(&ph[ks], hw, 16);
    __builtin_memcpy(&plo[ks], lw, 16);
    __builtin_memcpy(&vb[ks], &vv, 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's plane copies landed
  __syncthreads();                     // and every wave's, and g
  floatx16 dv[2], dk[2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[x][r] = dk[x][r] = 0.0f;
  const uint32_t base = lds_addr(smem);
  const int colq = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // dV: G rows 16 ks + 8 h2 .. +7 of column 32 (2 chalf + x) + l32, both planes
    uint32_t ad[8];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int r = 16 * ks + 8 * h2 + 4 * tt + (g16 >> 2);
          const int colb = 32 * (2 * chalf + x) + colq;
          ad[4 * x + 2 * pl + tt] =
              base + pl * PLANE + r * ROWB + 16 * ((colb >> 3) ^ swz(r)) + 2 * (colb & 7);
        }
    v4i16 fr[8];
    lds_read_tr<8>(fr, ad);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const bf16x8 gh = join_tr(fr[4 * x], fr[4 * x + 1]), gl = join_tr(fr[4 * x + 2], fr[4 * x + 3]);
      dv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[ks], gh, dv[x], 0, 0, 0);
      dv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(plo[ks], gh, dv[x], 0, 0, 0);
      dv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[ks], gl, dv[x], 0, 0, 0);
    }
    // dK^T: G row 32 (2 chalf + x) + l32, channels 16 ks + 8 h2 .. +7, both planes
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int a = 32 * (2 * chalf + x) + l32;
      const int ofs = a * ROWB + 16 * ((2 * ks + h2) ^ swz(a));
      const bf16x8 gh = lds_read16(smem + ofs), gl = lds_read16(smem + PLANE + ofs);
      dk[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, vb[ks], dk[x], 0, 0, 0);
      dk[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gl, vb[ks], dk[x], 0, 0, 0);
    }
  }
  // dV: lane holds keys 32 ut + 8 (r / 4) + 4 h2 + r % 4 of column 32 (2 chalf + x) + l32
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int u = key0 + 32 * ut + 8 * (r >> 2) + 4 * h2 + (r & 3);
      if (u < N) dvl[head + (size_t)u * D + 32 * (2 * chalf + x) + l32] = dv[x][r];
    }
  // dK: lane holds channels 32 (2 chalf + x) + 8 g + 4 h2 .. +3 of key urow
  if (ulive) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = 32 * (2 * chalf + x) + 8 * g + 4 * h2;
        const uint2 kk = *reinterpret_cast<const uint2*>(k + head + (size_t)urow * D + a0);
        const float kf[4] = {bf16_lo(kk.x), bf16_hi(kk.x), bf16_lo(kk.y), bf16_hi(kk.y)};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = elu1(kf[e]);
          y[e] = (dk[x][4 * g + e] + gs[a0 + e]) * (f > 1.0f ? 1.0f : f);
        }
        *reinterpret_cast<float4*>(dkl + head + (size_t)urow * D + a0) =
            make_float4(y[0], y[1], y[2], y[3]);
      }
  }
}

// dO_s = alpha (*) dO (the mix's sparse share), bf16; one thread per 8 values.
template <int D>
__global__ __launch_bounds__(256) void scale_do_kernel(const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ alpha,
                                                       uint16_t* __restrict__ dos, int H, int N,
                                                       size_t n8) {
  const size_t p = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= n8) return;
  const size_t e = p * 8;
  const int h = (int)((e / ((size_t)N * D)) % H), c = (int)(e % D);
  const uint4 u = *reinterpret_cast<const uint4*>(dO + e);
  const uint32_t* w = &u.x;
  uint4 o;
  uint32_t* ow = &o.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ow[i] = pack2_bf16(alpha[(size_t)h * D + c + 2 * i] * bf16_lo(w[i]),
                       alpha[(size_t)h * D + c + 2 * i + 1] * bf16_hi(w[i]));
  *reinterpret_cast<uint4*>(dos + e) = o;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* __restrict__ p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    p[e] = 0;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace regions, in order (the linear ones only when the branch is on)
struct BwdWs {
  uint16_t* kt;
  float *drow, *lse2;
  int32_t *cmat, *colcnt, *coloff, *collist;
  // linear branch
  uint16_t *vtp, *dos, *hj, *hd, *dhp, *gp;
  uint32_t *mbits, *mtbits;
  float *zd, *gz;
  int32_t *lin_on, *lin_lists;
  float *dql, *dkl, *dvl;
};

BwdWs bwd_layout(unsigned char* w, int B, int H, int N, int d, int block_q, bool linear,
                 size_t* bytes) {
  const size_t BH = (size_t)B * H, n_q = (N + block_q - 1) / block_q, n_k = (N + BK - 1) / BK;
  const size_t packed = BH * n_k * BK * d * 2, rows = BH * N * d;
  BwdWs r{};
  size_t off = 0;
  auto take = [&](size_t n) {
    unsigned char* p = w ? w + off : nullptr;
    off += up256(n);
    return p;
  };
  r.kt = reinterpret_cast<uint16_t*>(take(packed));
  r.drow = reinterpret_cast<float*>(take(BH * n_q * block_q * 4));  // rows padded to whole blocks
  r.lse2 = reinterpret_cast<float*>(take(BH * n_q * block_q * 4));
  r.cmat = reinterpret_cast<int32_t*>(take(BH * n_k * n_q * 4));
  r.colcnt = reinterpret_cast<int32_t*>(take(BH * n_k * 4));
  r.coloff = reinterpret_cast<int32_t*>(take(BH * (n_k + 1) * 4));
  r.collist = reinterpret_cast<int32_t*>(take(BH * n_q * n_k * 4));
  if (linear) {
    const size_t cols = (size_t)d * d + d, n_kw = (n_k + 31) / 32, n_qw = (n_q + 31) / 32;
    r.vtp = reinterpret_cast<uint16_t*>(take(packed));
    r.dos = reinterpret_cast<uint16_t*>(take(rows * 2));
    r.hj = reinterpret_cast<uint16_t*>(take(BH * n_k * 2 * cols * 2));
    r.mbits = reinterpret_cast<uint32_t*>(take(BH * n_q * n_kw * 4));
    r.hd = reinterpret_cast<uint16_t*>(take(BH * n_q * 2 * (size_t)d * d * 2));
    r.zd = reinterpret_cast<float*>(take(BH * n_q * d * 4));
    r.dhp = reinterpret_cast<uint16_t*>(take(BH * n_q * 2 * cols * 2));
    r.mtbits = reinterpret_cast<uint32_t*>(take(BH * n_k * n_qw * 4));
    r.gp = reinterpret_cast<uint16_t*>(take(BH * n_k * 2 * (size_t)d * d * 2));
    r.gz = reinterpret_cast<float*>(take(BH * n_k * d * 4));
    r.lin_on = reinterpret_cast<int32_t*>(take(H * 4));
    r.lin_lists = reinterpret_cast<int32_t*>(take((2 + 2 * BH) * 4));
    r.dql = reinterpret_cast<float*>(take(rows * 4));
    r.dkl = reinterpret_cast<float*>(take(rows * 4));
    r.dvl = reinterpret_cast<float*>(take(rows * 4));
  }
  if (bytes) *bytes = off;
  return r;
}

template <int D, int BQ>
hipError_t launch_bwd_t(const BwdLaunch& a, hipStream_t s) {
  const bool linear = a.alpha != nullptr;
  const BwdWs w = bwd_layout(a.workspace, a.B, a.H, a.N, a.d, a.block_q, linear, nullptr);
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  const uint16_t* dos = a.dO;  // the sparse part's upstream gradient
  if (linear) {
    if constexpr (D == BQ) {
      hipLaunchKernelGGL(linear_flags_kernel, dim3(1), dim3(kFlagThreads), 0, s, a.alpha,
                         a.lin_mode, D, a.drop_below, a.B, a.H, w.lin_on, w.lin_lists);
      // H_D, z_D of every query block, as the forward forms them
      const int qrows = BH * a.n_q, n_kw = (a.n_k + 31) / 32;
      hipLaunchKernelGGL((linear_pack_kernel<D>), dim3(a.n_k, BH), dim3(2 * D), 0, s, a.v, a.k,
                         w.vtp, w.hj, a.N, a.n_k, w.lin_on, a.H);
      hipLaunchKernelGGL(linear_mdrop_kernel, dim3((qrows + 3) / 4), dim3(256), 0, s, a.idx,
                         a.cnt, w.mbits, a.n_k, n_kw, qrows);
      hipLaunchKernelGGL((linear_hd_kernel<D>),
                         dim3((lin_cols<D>() + 127) / 128, (a.n_q + 255) / 256, BH), dim3(256), 0,
                         s, w.hj, w.mbits, w.hd, w.zd, a.n_q, a.n_k, n_kw, w.lin_on, a.H);
      if (a.lin_mode == kLinMix) {
        const size_t n8 = (size_t)BH * a.N * D / 8;
        hipLaunchKernelGGL((scale_do_kernel<D>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                           s, a.dO, a.alpha, w.dos, a.H, a.N, n8);
        dos = w.dos;
      }
    }
  }
  // K^T (fp16) packed in 64-row groups like V^T
  hipLaunchKernelGGL((pack_kernel<D, true>), dim3(a.n_k, BH), dim3(2 * D), 0, s, a.k, w.kt, a.N,
                     a.n_k);
  const int NP = a.n_q * BQ;
  const size_t rows = (size_t)BH * NP;
  constexpr int RPW = 256 / (D / 8);
  // D = dO . O with the caller's dO and O (the linear kernel corrects it to the sparse share)
  hipLaunchKernelGGL((bwd_rows_kernel<D>), dim3((unsigned)((rows + RPW - 1) / RPW)), dim3(256), 0,
                     s, a.o, a.dO, a.lse, w.drow, w.lse2, a.N, NP, rows);
  // the query blocks that list each key block
  const size_t cm = (size_t)BH * a.n_k * a.n_q;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<size_t>((cm + 255) / 256, 4096)),
                     dim3(256), 0, s, w.cmat, cm);
  const int qrows = BH * a.n_q, cols = BH * a.n_k;
  hipLaunchKernelGGL(col_count_kernel, dim3((qrows + 3) / 4), dim3(256), 0, s, a.idx, a.cnt,
                     w.cmat, a.n_q, a.n_k, qrows);
  hipLaunchKernelGGL(col_total_kernel, dim3((cols + 3) / 4), dim3(256), 0, s, w.cmat, w.colcnt,
                     a.n_q, cols);
  hipLaunchKernelGGL(col_scan_kernel, dim3(BH), dim3(256), 0, s, w.colcnt, w.coloff, a.n_k);
  hipLaunchKernelGGL(col_list_kernel, dim3((cols + 3) / 4), dim3(256), 0, s, w.cmat, w.coloff,
                     w.collist, a.n_q, a.n_k, cols);
  if (linear) {
    if constexpr (D == BQ) {
      if constexpr (D == 128)
        hipLaunchKernelGGL((linear_bwd_rows_mfma_kernel<D>), dim3(qrows), dim3(256), 0, s, a.q,
                           a.dO, w.hd, w.zd, a.cnt, w.lin_on, a.alpha, a.lin_mode, w.dql, w.dhp,
                           w.drow, a.H, a.N, a.n_q, a.n_k, NP, qrows);
      else
        hipLaunchKernelGGL((linear_bwd_rows_kernel<D>), dim3(qrows), dim3(256), 0, s, a.q, a.dO,
                           w.hd, w.zd, a.cnt, w.lin_on, a.alpha, a.lin_mode, w.dql, w.dhp, w.drow,
                           a.H, a.N, a.n_q, a.n_k, NP, qrows);
      // G_j, g_j: the query blocks' dH_D, dz_D summed over those that dropped key block j
      const int n_kw = (a.n_k + 31) / 32, n_qw = (a.n_q + 31) / 32;
      const size_t words = (size_t)BH * a.n_k * n_qw;
      hipLaunchKernelGGL(linear_mtrans_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                         s, w.mbits, w.mtbits, a.n_q, a.n_k, n_kw, n_qw, BH);
      hipLaunchKernelGGL((linear_hd_kernel<D>),
                         dim3((lin_cols<D>() + 127) / 128, (a.n_k + 255) / 256, BH), dim3(256), 0,
                         s, w.dhp, w.mtbits, w.gp, w.gz, a.n_k, a.n_q, n_qw, w.lin_on, a.H);
      if constexpr (D == 128)
        hipLaunchKernelGGL((linear_bwd_keys_mfma_kernel<D>), dim3(cols), dim3(256), 0, s, a.k,
                           a.v, w.gp, w.gz, w.lin_on, w.dkl, w.dvl, a.H, a.N, a.n_k, cols);
      else
        hipLaunchKernelGGL((linear_bwd_keys_kernel<D>), dim3(cols), dim3(256), 0, s, a.k, a.v,
                           w.gp, w.gz, w.lin_on, w.dkl, w.dvl, a.H, a.N, a.n_k, cols);
    }
  }
  if constexpr (D == 128)
    hipLaunchKernelGGL((sparse_attn_bwd_dkdv8_kernel<BQ>), dim3(cols), dim3(512), 0, s, a.q, a.k,
                       a.v, dos, w.lse2, w.drow, w.coloff, w.collist, a.dk, a.dv, a.N, a.n_q,
                       a.n_k, cols, c, a.scale, linear ? w.dkl : nullptr, linear ? w.dvl : nullptr);
  else
    hipLaunchKernelGGL((sparse_attn_bwd_dkdv_kernel<D, BQ>), dim3(cols), dim3(256), 0, s, a.q,
                       a.k, a.v, dos, w.lse2, w.drow, w.coloff, w.collist, a.dk, a.dv, a.N, a.n_q,
                       a.n_k, cols, c, a.scale, linear ? w.dkl : nullptr, linear ? w.dvl : nullptr);
  hipLaunchKernelGGL((sparse_attn_bwd_dq_kernel<D, BQ>), dim3(qrows), dim3(BQ * 2), 0, s, a.q,
                     a.k, a.v, dos, w.kt, w.lse2, w.drow, a.idx, a.cnt, a.dq, a.N, a.n_q,
                     a.n_k, qrows, c, a.scale, linear ? w.dql : nullptr);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d, int block_q, bool linear) {
  size_t bytes = 0;
  bwd_layout(nullptr, B, H, N, d, block_q, linear, &bytes);
  return bytes;
}

hipError_t launch_bwd(const BwdLaunch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_bwd_t<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_bwd_t<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_bwd_t<64, 128>(a, s);
  return launch_bwd_t<64, 64>(a, s);
}

}  // namespace sparge
