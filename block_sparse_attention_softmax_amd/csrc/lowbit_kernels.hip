// Low-bit sparse branch (SLA2 page, section 2C: Q, K, P and V quantised in
// the forward pass of the sparse attention):
//
//   Q, K  INT8 codes, one float32 scale per block (query blocks of block_q
//         rows, key blocks of 64): scale = amax / 127, code = rint(x * 127/amax)
//   V     FP8 e4m3 (OCP e4m3fn) codes of x * 448/amax_c, one scale per
//         (head, channel)
//   P     e4m3 codes of 448 p, p = exp(scale (s - m)) against the exact
//         running row maximum m (so p <= 1), blocks in list order
//   O     = sum p~ v~ / sum p~
//
// S^T = K Q^T runs on v_mfma_i32_32x32x32_i8 (exact integer sums), the
// product O^T += V^T P^T on v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales
// (one instruction per 32 channels covers the block's 64 keys). As in the
// bf16 kernel, the transposed products keep one query per lane, and V^T is
// packed so that the P^T codes of a lane feed the B operand unchanged: for
// lane half h the 64-key operand index 32 h + i holds key
// 32 (i / 16) + 8 ((i % 16) / 4) + 4 h + i % 4, the key whose score register
// 16 (i / 16) + i % 16 of that lane holds.
#include <climits>

#include "internal.h"
#include "tiles.h"

namespace sparge {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr float kE4m3Max = 448.0f;

__global__ __launch_bounds__(256) void fill_u32_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0u;
}

// --------------------------------------------------------- quantisation
// INT8 codes of one block of rows of a [rows][D] bf16 array and its scale.
// One workgroup (256 threads) per (block, b*h).
template <int D>
__global__ __launch_bounds__(256) void quant_int8_kernel(const uint16_t* __restrict__ x,
                                                         int8_t* __restrict__ codes,
                                                         float* __restrict__ scales, int N,
                                                         int block, int nblocks) {
  __shared__ float red[4];
  const int bi = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int r0 = bi * block, rows = min(block, N - r0);
  const size_t base = ((size_t)bh * N + r0) * D;
  const int n8 = rows * D / 8;
  // the block (at most 128 rows) stays in registers between its amax and its codes
  constexpr int MAXU = 128 * D / 8 / 256;
  uint4 u[MAXU];
#pragma unroll
  for (int q8 = 0; q8 < MAXU; ++q8) {
    const int p = q8 * 256 + t;
    u[q8] = p < n8 ? *reinterpret_cast<const uint4*>(x + base + (size_t)p * 8) : make_uint4(0, 0, 0, 0);
  }
  float amax = 0.0f;
#pragma unroll
  for (int q8 = 0; q8 < MAXU; ++q8) {
    const uint32_t* w = &u[q8].x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (t == 0) scales[(size_t)bh * nblocks + bi] = amax / 127.0f;
#pragma unroll
  for (int q8 = 0; q8 < MAXU; ++q8) {
    const int p = q8 * 256 + t;
    if (p < n8)
      *reinterpret_cast<uint2*>(codes + base + (size_t)p * 8) =
          make_uint2(int8_pack4(u[q8].x, u[q8].y, inv), int8_pack4(u[q8].z, u[q8].w, inv));
  }
}

// amax over the rows of each channel of V: as float bits (non-negative floats
// order like their bits), max-combined into vmax[bh][c], which starts at 0.
// Grid (chunks of kAmaxRows rows, b*h), 256 threads: D/8 threads cover a row
// with 16-byte loads, 256/(D/8) rows at a time; the row lanes meet through LDS.
constexpr int kAmaxRows = 256;
template <int D>
__global__ __launch_bounds__(256) void v_amax_kernel(const uint16_t* __restrict__ v,
                                                     uint32_t* __restrict__ vmax, int N) {
  constexpr int CG = D / 8, RL = 256 / CG;  // channel groups, row lanes
  __shared__ float part[RL][D];
  const int bh = blockIdx.y, t = threadIdx.x, cg = t % CG, rl = t / CG;
  const int r0 = blockIdx.x * kAmaxRows, r1 = min(r0 + kAmaxRows, N);
  float mx[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int UNR = 8;  // rows in flight per thread (their loads issued together)
  for (int rb = r0 + rl; rb < r1; rb += RL * UNR) {
    uint4 u[UNR];
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      const int r = min(rb + RL * x, r1 - 1);  // a repeated row leaves the maximum unchanged
      u[x] = *reinterpret_cast<const uint4*>(v + ((size_t)bh * N + r) * D + 8 * cg);
    }
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      const uint32_t* w = &u[x].x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mx[2 * e] = fmaxf(mx[2 * e], fabsf(bf16_lo(w[e])));
        mx[2 * e + 1] = fmaxf(mx[2 * e + 1], fabsf(bf16_hi(w[e])));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rl][8 * cg + e] = mx[e];
  __syncthreads();
  if (t < D) {
    float m = 0.0f;
#pragma unroll
    for (int l = 0; l < RL; ++l) m = fmaxf(m, part[l][t]);
    atomicMax(&vmax[(size_t)bh * D + t], __float_as_uint(m));
  }
}

// Slot of the packed fp8 V^T block (see the file comment) -> key.
__device__ __forceinline__ int fp8_slot_key(int slot) {
  const int h = slot >> 5, i = slot & 31;
  return 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * h + (i & 3);
}

// vt8[bh][j][c][slot] = e4m3(V[bh][64 j + key(slot)][c] * 448 / amax_c), zero
// past N. Grid (key blocks, b*h), 256 threads: the 64 V rows are staged in
// LDS with 16-byte loads, then each thread writes 4-byte groups of slots of
// one channel row.
template <int D>
__global__ __launch_bounds__(256) void pack_v_fp8_kernel(const uint16_t* __restrict__ v,
                                                         const uint32_t* __restrict__ vmax,
                                                         uint8_t* __restrict__ vt8, int N,
                                                         int n_k) {
  __shared__ uint16_t vs[BK * (D + 2)];  // rows padded by one word against bank conflicts
  __shared__ float sinv[D];               // 448 / amax per channel
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  constexpr int LU = BK * D / 8 / 256;  // 16-byte loads per thread, issued together
  static_assert(BK * D / 8 % 256 == 0, "whole loads per thread");
  uint4 u[LU];
#pragma unroll
  for (int x = 0; x < LU; ++x) {
    const int p = x * 256 + t, r = p / (D / 8), c8 = (p % (D / 8)) * 8;
    u[x] = make_uint4(0, 0, 0, 0);
    if (j * BK + r < N) u[x] = *reinterpret_cast<const uint4*>(v + ((size_t)bh * N + j * BK + r) * D + c8);
  }
  if (t < D) {
    const float amax = __uint_as_float(vmax[(size_t)bh * D + t]);
    sinv[t] = amax > 0.0f ? kE4m3Max / amax : 0.0f;
  }
#pragma unroll
  for (int x = 0; x < LU; ++x) {
    const int p = x * 256 + t, r = p / (D / 8), c8 = (p % (D / 8)) * 8;
    const uint32_t* w = &u[x].x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vs[r * (D + 2) + c8 + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      vs[r * (D + 2) + c8 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  for (int p = t; p < D * 16; p += 256) {
    const int c = p / 16, s0 = (p % 16) * 4;
    const float inv = sinv[c];
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = __uint_as_float((uint32_t)vs[fp8_slot_key(s0 + e) * (D + 2) + c] << 16) * inv;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
    *reinterpret_cast<int*>(vt8 + (((size_t)bh * n_k + j) * D + c) * BK + s0) = w;
  }
}

// ------------------------------------------------------------ attention
// LDS tiles: K codes [64 keys][D bytes] and packed V^T codes [D][64 bytes],
// 16-byte chunks XOR-swizzled so that the 32 rows an operand read touches
// cover all banks: rows of R bytes share a 256-byte bank window 256 / R at a
// time, so chunk c of row r is stored at c ^ ((r / (256 / R)) mod (R / 16)).
template <int R>
struct Tile8 {
  static constexpr int CPR = R / 16;          // chunks per row
  static constexpr int RPW = 256 / R;         // rows per bank window
  static constexpr int BYTES = 64 * R;        // K tile (64 rows); V^T tile has D rows of 64 bytes
  __device__ static constexpr int swz(int row, int chunk) { return chunk ^ ((row / RPW) & (CPR - 1)); }
};

// Three workgroups per CU (168 registers per wave at BQ = 128): the kernel is
// bound by its softmax VALU work, so a third wave per SIMD to interleave pays
// more than a deeper pipeline within a wave would (4% measured over two).
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 3) void sparse_attn_lowbit_kernel(
    const int8_t* __restrict__ qc, const float* __restrict__ qs, const int8_t* __restrict__ kc,
    const float* __restrict__ ks, const uint8_t* __restrict__ vt8,
    const uint32_t* __restrict__ vmax, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ o, int N, int n_q, int n_k,
    int total, float c) {
  using TK = Tile8<D>;   // K rows: D bytes
  using TV = Tile8<BK>;  // V^T rows: 64 bytes
  constexpr int NT = BQ * 2, DT = D / 32, KS = D / 32;
  constexpr int KBYTES = BK * D, VBYTES = D * BK;
  constexpr int KU = KBYTES / 16 / NT, VU = VBYTES / 16 / NT;  // 16-byte copies per thread
  static_assert(KBYTES % (16 * NT) == 0 && VBYTES % (16 * NT) == 0, "whole copies per thread");
  __shared__ __align__(16) unsigned char smem[2 * (KBYTES + VBYTES)];

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const int qrow = qi * BQ + wave * 32 + l32;

  v4i qf[KS];  // Q codes of this lane's query, d = 32 s + 16 h2 .. +15
  {
    const int8_t* qp = qc + head + (size_t)min(qrow, N - 1) * D + 16 * h2;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const v4i*>(qp + 32 * s);
  }
  const float sq = qs[(size_t)bh * n_q + qi];
  const int count = min(max(kv_cnt[tile], 0), n_k);
  const int32_t* ids = kv_idx + (size_t)tile * n_k;
  auto jat = [&](int e) { return min(max(ids[e], 0), n_k - 1); };

  // per-thread copy offsets within a tile
  uint32_t ksrc[KU], vsrc[VU];
  int krow[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int p = u * NT + threadIdx.x, r = p / TK::CPR;
    krow[u] = r;
    ksrc[u] = (uint32_t)(r * D + TK::swz(r, p % TK::CPR) * 16);
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = u * NT + threadIdx.x, r = p / TV::CPR;
    vsrc[u] = (uint32_t)(r * BK + TV::swz(r, p % TV::CPR) * 16);
  }
  auto issue = [&](int j, int b) {  // K rows past N read row N - 1 (masked below)
    const int key0 = j * BK;
    const int8_t* kb = kc + head + (size_t)key0 * D;
    const uint8_t* vb = vt8 + ((size_t)bh * n_k + j) * VBYTES;
    unsigned char* kd = smem + b * (KBYTES + VBYTES);
    unsigned char* vd = kd + KBYTES;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t back = (uint32_t)max(key0 + krow[u] - (N - 1), 0) * D;
      dma16(kb + ksrc[u] - back, kd + (u * NT + wave * 64) * 16);
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) dma16(vb + vsrc[u], vd + (u * NT + wave * 64) * 16);
  };

  floatx16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m = -INFINITY;  // running max of s
  // The sum of the P codes' values comes from one more FP8 product: an A
  // operand of e4m3 ones (0x38) gives, in every register of every lane, the
  // sum over the block's 64 keys of that lane's query (instead of decoding the
  // codes on the VALU); register 0 is kept.
  constexpr int one8 = 0x38383838;
  const v8i ones = {one8, one8, one8, one8, one8, one8, one8, one8};
  floatx16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;

  if (count > 0) issue(jat(0), 0);
  for (int e = 0; e < count; ++e) {
    const int j = jat(e);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of block e landed
    __syncthreads();                     // all copies landed; the other buffer is free
    if (e + 1 < count) issue(jat(e + 1), (e + 1) & 1);
    const unsigned char* kt = smem + (e & 1) * (KBYTES + VBYTES);
    const unsigned char* vtl = kt + KBYTES;

    // S^T = K Q^T in exact integers, then s = dot * (sq sk) in float32
    v16i si[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int r = 0; r < 16; ++r) si[tau][r] = 0;
      const int kr = 32 * tau + l32;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v4i a = *reinterpret_cast<const v4i*>(kt + kr * D + TK::swz(kr, 2 * s + h2) * 16);
        si[tau] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], si[tau], 0, 0, 0);
      }
    }
    // s = dot * (sq sk): the row maximum is taken on the integers (the scale is
    // positive), and 448 p = 2^(dot (sq sk c) - m c + log2 448) in one FMA
    const float sqk = sq * ks[(size_t)bh * n_k + j];
    const int nvalid = N - j * BK;  // keys past N (last block only) take no part
    if (nvalid < BK) {              // a ragged last block: a uniform branch, taken once per row
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * tau + 8 * (r >> 2) + 4 * h2 + (r & 3) >= nvalid) si[tau][r] = INT_MIN;
    }
    int dmax = INT_MIN;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; r += 2) dmax = max(dmax, max(si[tau][r], si[tau][r + 1]));
    dmax = max(dmax, __shfl_xor(dmax, 32));
    const float mloc = (float)dmax * sqk;
    const float m_new = fmaxf(m, mloc);
    if (__any(m_new > m)) {  // exact running maximum: rescale whenever it rises
      const float f = m_new > m ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.0f;
      lacc[0] *= f;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= f;
      m = m_new;
    }
    // P codes: e4m3(448 p), four per dword, in register order (word w holds
    // keys 32 (w / 4) + 8 (w % 4) + 4 h2 + 0..3)
    v8i pb;
    const float sc = sqk * c, bias = 8.807354922057604f - m * c;  // log2(448) - m c
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int tau = w >> 2, r0 = (w & 3) * 4;
      float p[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        p[e2] = __builtin_amdgcn_exp2f(fmaf((float)si[tau][r0 + e2], sc, bias));
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      pb[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
    }
    if (nvalid < BK) {  // masked keys get code 0 (byte-wise, keys ascend within a word)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int nv = min(max(nvalid - (32 * (w >> 2) + 8 * (w & 3) + 4 * h2), 0), 4);
        pb[w] &= nv >= 4 ? -1 : (int)((1u << (8 * nv)) - 1u);
      }
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, lacc, 0, 0, 0, 127, 0, 127);
    // O^T += V^T P^T, one instruction per 32 channels covers the 64 keys
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      const int row = 32 * i + l32;
      const v4i a0 = *reinterpret_cast<const v4i*>(vtl + row * BK + TV::swz(row, 2 * h2) * 16);
      const v4i a1 = *reinterpret_cast<const v4i*>(vtl + row * BK + TV::swz(row, 2 * h2 + 1) * 16);
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      oacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[i], 0, 0, 0, 127, 0,
                                                                 127);
    }
  }

  // O = sv_c * sum(codeP codeV) / sum(codeP) (the 448s cancel)
  const float ltot = lacc[0];
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  // O leaves through LDS as whole rows (each wave's 32 x D tile in its own
  // slice of the tile buffers, free once every wave is past its last block)
  static_assert(BQ * D * 2 <= (int)sizeof(smem), "the O tiles must fit the tile buffers");
  __syncthreads();
  store_rows_via_lds<D>(smem + wave * 32 * D * 2, o + head, qi * BQ + wave * 32, N, lane,
                        [&](int i, int g) {
                          const int d0 = 32 * i + 8 * g + 4 * h2;
                          float y[4];
#pragma unroll
                          for (int e2 = 0; e2 < 4; ++e2) {
                            const float sv_c =
                                __uint_as_float(vmax[(size_t)bh * D + d0 + e2]) / kE4m3Max;
                            y[e2] = oacc[i][4 * g + e2] * sv_c * inv;
                          }
                          uint2 pk;
                          pk.x = pack2_bf16(y[0], y[1]);
                          pk.y = pack2_bf16(y[2], y[3]);
                          return pk;
                        });
}

template <int D, int BQ>
hipError_t launch_lowbit_t(const LowbitLaunch& a, hipStream_t s) {
  const int BH = a.B * a.H, total = BH * a.n_q;
  if (a.phase == kLowbitAll) {
    hipLaunchKernelGGL((quant_int8_kernel<D>), dim3(a.n_q, BH), dim3(256), 0, s, a.q, a.qc, a.qs,
                       a.N, BQ, a.n_q);
    hipLaunchKernelGGL((quant_int8_kernel<D>), dim3(a.n_k, BH), dim3(256), 0, s, a.k, a.kc, a.ks,
                       a.N, BK, a.n_k);
  }
  if (a.phase != kLowbitAttend) {
    const size_t nv = (size_t)BH * D;
    hipLaunchKernelGGL(fill_u32_zero_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, s,
                       a.vmax, nv);
    hipLaunchKernelGGL((v_amax_kernel<D>), dim3((a.N + kAmaxRows - 1) / kAmaxRows, BH), dim3(256),
                       0, s, a.v, a.vmax, a.N);
    hipLaunchKernelGGL((pack_v_fp8_kernel<D>), dim3(a.n_k, BH), dim3(256), 0, s, a.v, a.vmax,
                       a.vt8, a.N, a.n_k);
    if (a.phase == kLowbitPackV) return hipGetLastError();
  }
  hipLaunchKernelGGL((sparse_attn_lowbit_kernel<D, BQ>), dim3(total), dim3(BQ * 2), 0, s, a.qc,
                     a.qs, a.kc, a.ks, a.vt8, a.vmax, a.idx, a.cnt, a.o, a.N, a.n_q, a.n_k, total,
                     a.scale * 1.4426950408889634f);
  return hipGetLastError();
}

}  // namespace

size_t lowbit_workspace_bytes(int B, int H, int N, int d, int block_q) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)B * H, n_q = (N + block_q - 1) / block_q, n_k = (N + BK - 1) / BK;
  return 2 * up(BH * N * d) + up(BH * n_q * 4) + up(BH * n_k * 4) + up(BH * d * 4) +
         up(BH * n_k * BK * d);
}

void lowbit_layout(LowbitLaunch& a, unsigned char* w) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)a.B * a.H;
  size_t off = 0;
  a.qc = reinterpret_cast<int8_t*>(w + off);
  off += up(BH * a.N * a.d);
  a.kc = reinterpret_cast<int8_t*>(w + off);
  off += up(BH * a.N * a.d);
  a.qs = reinterpret_cast<float*>(w + off);
  off += up(BH * a.n_q * 4);
  a.ks = reinterpret_cast<float*>(w + off);
  off += up(BH * a.n_k * 4);
  a.vmax = reinterpret_cast<uint32_t*>(w + off);
  off += up(BH * a.d * 4);
  a.vt8 = w + off;
}

hipError_t launch_lowbit(const LowbitLaunch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_lowbit_t<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_lowbit_t<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_lowbit_t<64, 128>(a, s);
  return launch_lowbit_t<64, 64>(a, s);
}

}  // namespace sparge
