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
//    to bf16, feed the second products as B operands unchanged, against Q^T
//    and dO^T pre-packed in the same slot order as the forward's V^T.
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
// lse2[bh][t] = lse[bh][t] * log2(e), in rows padded to NP = 64 * ceil(N / 64)
// per (b, h) so that whole 64-row groups can be copied: padding rows get
// D = 0 and lse2 = +inf (P = 0). D/8 lanes per row.
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
// of the block (one per lane % 32) and takes queries 32*(w >> 1) .. +31 of
// every 64-query stage; the two query halves are summed at the end.
//
// A stage (Q rows, dO rows, packed Q^T and dO^T of one 64-row group, and its
// lse2 and D) is copied global -> LDS by direct-to-LDS loads into one of two
// buffers while the waves compute on the other. Lane i of a wave's copy lands
// at LDS base + 16 i, so each lane reads the global chunk that the tile's XOR
// swizzle puts there; rows past N read row N - 1 instead (their lse2 is +inf,
// so they contribute P = dS = 0).
template <int D>
struct DkdvStage {
  using T = Tile<D>;
  static constexpr int BYTES = 4 * T::BYTES + 2 * 64 * 4;
  static constexpr int QS = 0, DS = T::BYTES, QTS = 2 * T::BYTES, DTS = 3 * T::BYTES,
                       LS = 4 * T::BYTES, DD = 4 * T::BYTES + 256;
};

__device__ __forceinline__ void dma4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

template <int D, int BQ>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void sparse_attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ qt, const uint16_t* __restrict__ dot,
    const float* __restrict__ lse2, const float* __restrict__ drow,
    const int32_t* __restrict__ coloff, const int32_t* __restrict__ collist,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int n_q, int n_k, int n64,
    int total, float c, float scale) {
  using T = Tile<D>;
  using ST = DkdvStage<D>;
  constexpr int DT = D / 32, KSTEPS = D / 16, SUB = BQ / 64;
  constexpr int KU = 64 * T::KCPR / 256, VU = D * T::VCPR / 256;  // 16-byte copies per thread
  __shared__ __align__(16) unsigned char smem[2 * ST::BYTES];

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_k, j = tile % n_k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // copy bases are uniform
  const int h2 = lane >> 5, l32 = lane & 31, kw = 32 * (wave & 1), qh = wave >> 1;
  const size_t head = (size_t)bh * N * D;
  const int NP = n64 * BK;
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

  // per-thread source offsets (elements) of the tile copies, within a row group
  uint32_t krow_ofs[KU], vrow_ofs[VU];
  int krow[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int p = u * 256 + threadIdx.x, r = p / T::KCPR;
    krow[u] = r;
    krow_ofs[u] = (uint32_t)(r * D + T::kchunk(r, p % T::KCPR) * 8);
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = u * 256 + threadIdx.x, r = p / T::VCPR;
    vrow_ofs[u] = (uint32_t)(r * BK + T::vchunk(r, p % T::VCPR) * 8);
  }

  const int beg = coloff[(size_t)bh * (n_k + 1) + j], end = coloff[(size_t)bh * (n_k + 1) + j + 1];
  const int32_t* lst = collist + (size_t)bh * n_q * n_k;
  // stages: (entry e, sub-block sb) with row r0 = lst[e] * BQ + 64 sb < N
  auto first_row = [&](int e, int sb) { return lst[e] * BQ + 64 * sb; };
  auto advance = [&](int& e, int& sb) {  // to the next stage that starts before N
    do {
      if (++sb == SUB) {
        sb = 0;
        ++e;
      }
    } while (e < end && first_row(e, sb) >= N);
  };
  auto issue = [&](int r0, unsigned char* buf) {
    const uint16_t* qsrc = q + head + (size_t)r0 * D;
    const uint16_t* dsrc = dO + head + (size_t)r0 * D;
    const size_t g = (size_t)bh * n64 + r0 / 64;
    const uint16_t* qtsrc = qt + g * D * BK;
    const uint16_t* dtsrc = dot + g * D * BK;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t back = (uint32_t)max(r0 + krow[u] - (N - 1), 0) * D;  // rows past N
      unsigned char* dst = buf + (u * 256 + wave * 64) * 16;
      dma16(qsrc + krow_ofs[u] - back, dst + ST::QS);
      dma16(dsrc + krow_ofs[u] - back, dst + ST::DS);
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      unsigned char* dst = buf + (u * 256 + wave * 64) * 16;
      dma16(qtsrc + vrow_ofs[u], dst + ST::QTS);
      dma16(dtsrc + vrow_ofs[u], dst + ST::DTS);
    }
    if (wave == 0) dma4(lse2 + (size_t)bh * NP + r0 + lane, buf + ST::LS);
    if (wave == 1) dma4(drow + (size_t)bh * NP + r0 + lane, buf + ST::DD);
  };

  int e = beg, sb = 0;
  if (e < end && first_row(e, sb) >= N) advance(e, sb);
  int it = 0;
  if (e < end) issue(first_row(e, sb), smem);
  while (e < end) {
    unsigned char* const buf = smem + (it & 1) * ST::BYTES;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of the stage landed
    __syncthreads();                     // every wave's copies landed, the other buffer is free
    int en = e, sn = sb;
    advance(en, sn);
    if (en < end) issue(first_row(en, sn), smem + ((it + 1) & 1) * ST::BYTES);

    const unsigned char* qs = buf + ST::QS;
    const unsigned char* ds = buf + ST::DS;
    const unsigned char* qts = buf + ST::QTS;
    const unsigned char* dts = buf + ST::DTS;
    const float* ls = reinterpret_cast<const float*>(buf + ST::LS);
    const float* dd = reinterpret_cast<const float*>(buf + ST::DD);

    // S = Q K^T and dP = dO V^T for the wave's 32 queries x 32 keys
    floatx16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
    const int qr = qh * 32 + l32;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int ch = 2 * s + h2;
      const bf16x8 a = lds_read16(qs + qr * T::KROWB + T::kchunk(qr, ch) * 16);
      const bf16x8 b = lds_read16(ds + qr * T::KROWB + T::kchunk(qr, ch) * 16);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[s], S, 0, 0, 0);
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, vf[s], dP, 0, 0, 0);
    }
    // P = 2^(S c - lse2), dS = P (dP - D); register r holds query
    // 8*(r/4) + 4*h2 + r%4 of the wave's 32
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int t0 = qh * 32 + 8 * gg + 4 * h2;
      const float4 l4 = *reinterpret_cast<const float4*>(ls + t0);
      const float4 d4 = *reinterpret_cast<const float4*>(dd + t0);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int r = 4 * gg + e2;
        const float p = __builtin_amdgcn_exp2f(fmaf(S[r], c, -lv[e2]));
        S[r] = p;
        dP[r] = p * (dP[r] - dv4[e2]);
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS (k = the wave's queries, in slot order)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pb = pack_bf16x8(S, 8 * t);
      const bf16x8 sb2 = pack_bf16x8(dP, 8 * t);
      const int ch = 4 * qh + 2 * t + h2;
#pragma unroll
      for (int ii = 0; ii < DT; ++ii) {
        const int row = 32 * ii + l32;
        const bf16x8 ao = lds_read16(dts + row * T::VROWB + T::vchunk(row, ch) * 16);
        const bf16x8 aq = lds_read16(qts + row * T::VROWB + T::vchunk(row, ch) * 16);
        dva[ii] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb, dva[ii], 0, 0, 0);
        dka[ii] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb2, dka[ii], 0, 0, 0);
      }
    }
    e = en;
    sb = sn;
    ++it;
  }

  // sum the two query halves: waves 2, 3 hand theirs to waves 0, 1
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [2 key halves][2][DT][16][64]
  static_assert(2 * 2 * DT * 16 * 64 * 4 <= 2 * DkdvStage<D>::BYTES, "reduction must fit");
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
    int total, float c, float scale) {
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
  const int NP = 64 * ((N + 63) / 64);
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
  if (valid) {
    uint16_t* orow = dq + head + (size_t)qrow * D;
#pragma unroll
    for (int ii = 0; ii < DT; ++ii)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d0 = 32 * ii + 8 * gg + 4 * h2;
        uint2 pk;
        pk.x = pack2_bf16(scale * acc[ii][4 * gg + 0], scale * acc[ii][4 * gg + 1]);
        pk.y = pack2_bf16(scale * acc[ii][4 * gg + 2], scale * acc[ii][4 * gg + 3]);
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* __restrict__ p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    p[e] = 0;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace regions, in order
struct BwdWs {
  uint16_t *qt, *dot, *kt;
  float *drow, *lse2;
  int32_t *cmat, *colcnt, *coloff, *collist;
};

BwdWs bwd_layout(unsigned char* w, int B, int H, int N, int d, int block_q, size_t* bytes) {
  const size_t BH = (size_t)B * H, n_q = (N + block_q - 1) / block_q, n_k = (N + BK - 1) / BK;
  const size_t packed = up256(BH * n_k * BK * d * 2);
  BwdWs r{};
  size_t off = 0;
  auto take = [&](size_t n) {
    unsigned char* p = w ? w + off : nullptr;
    off += up256(n);
    return p;
  };
  r.qt = reinterpret_cast<uint16_t*>(take(packed));
  r.dot = reinterpret_cast<uint16_t*>(take(packed));
  r.kt = reinterpret_cast<uint16_t*>(take(packed));
  r.drow = reinterpret_cast<float*>(take(BH * n_k * BK * 4));  // padded rows
  r.lse2 = reinterpret_cast<float*>(take(BH * n_k * BK * 4));
  r.cmat = reinterpret_cast<int32_t*>(take(BH * n_k * n_q * 4));
  r.colcnt = reinterpret_cast<int32_t*>(take(BH * n_k * 4));
  r.coloff = reinterpret_cast<int32_t*>(take(BH * (n_k + 1) * 4));
  r.collist = reinterpret_cast<int32_t*>(take(BH * n_q * n_k * 4));
  if (bytes) *bytes = off;
  return r;
}

template <int D, int BQ>
hipError_t launch_bwd_t(const BwdLaunch& a, hipStream_t s) {
  const BwdWs w = bwd_layout(a.workspace, a.B, a.H, a.N, a.d, a.block_q, nullptr);
  const int BH = a.B * a.H, n64 = a.n_k;  // 64-row groups of Q and dO = key blocks
  const float c = a.scale * kLog2e;
  // Q^T, dO^T and K^T (fp16) packed in 64-row groups like V^T
  hipLaunchKernelGGL((pack_kernel<D, false>), dim3(n64, BH), dim3(2 * D), 0, s, a.q, nullptr,
                     w.qt, nullptr, a.N, n64, nullptr, a.H);
  hipLaunchKernelGGL((pack_kernel<D, false>), dim3(n64, BH), dim3(2 * D), 0, s, a.dO, nullptr,
                     w.dot, nullptr, a.N, n64, nullptr, a.H);
  hipLaunchKernelGGL((pack_kernel<D, false, true>), dim3(n64, BH), dim3(2 * D), 0, s, a.k,
                     nullptr, w.kt, nullptr, a.N, n64, nullptr, a.H);
  const int NP = n64 * BK;
  const size_t rows = (size_t)BH * NP;
  constexpr int RPW = 256 / (D / 8);
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
  hipLaunchKernelGGL((sparse_attn_bwd_dkdv_kernel<D, BQ>), dim3(cols), dim3(256), 0, s, a.q, a.k,
                     a.v, a.dO, w.qt, w.dot, w.lse2, w.drow, w.coloff, w.collist, a.dk, a.dv,
                     a.N, a.n_q, a.n_k, n64, cols, c, a.scale);
  hipLaunchKernelGGL((sparse_attn_bwd_dq_kernel<D, BQ>), dim3(qrows), dim3(BQ * 2), 0, s, a.q,
                     a.k, a.v, a.dO, w.kt, w.lse2, w.drow, a.idx, a.cnt, a.dq, a.N, a.n_q,
                     a.n_k, qrows, c, a.scale);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d, int block_q) {
  size_t bytes = 0;
  bwd_layout(nullptr, B, H, N, d, block_q, &bytes);
  return bytes;
}

hipError_t launch_bwd(const BwdLaunch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_bwd_t<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_bwd_t<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_bwd_t<64, 128>(a, s);
  return launch_bwd_t<64, 64>(a, s);
}

}  // namespace sparge
