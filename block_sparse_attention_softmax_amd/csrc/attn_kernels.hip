// Block-sparse FlashAttention forward for gfx950 (SpargeAttention2 page,
// section 2C: tiles of Q/K/V, a block-level mask, and the masked tiles'
// matrix products and softmax skipped entirely).
//
// One workgroup per (batch, head, query block of BQ rows); BQ/32 waves, each
// owning 32 query rows. For every key block j listed for the row:
//
//   S^T (64 keys x 32 queries) = K_j Q^T     bf16 MFMA 32x32x16, fp32 acc
//   online softmax per query in fp32, base-2 exponent with scale*log2(e)
//   O^T (d x 32 queries) += V_j^T P^T        bf16 MFMA 32x32x16, fp32 acc
//
// Computing the transposed products puts one query per lane (lane % 32) in
// the MFMA output layout, so row maxima and sums need only one exchange
// between the two half-waves, and the rescaling of O uses the lane's own
// factor. The P^T accumulator registers are fed back as the B operand of the
// second product unchanged; V is pre-packed once per call (vt_pack_kernel)
// into key-contiguous tiles in the key order those registers imply, so both
// MFMA A operands are plain 16-byte LDS reads.
//
// K_j and packed V_j tiles are copied global -> LDS by direct-to-LDS loads,
// double-buffered: the copies of block j+1 are issued right after the
// barrier that opens block j and overlap all of block j's work.
#include "internal.h"

namespace sparge {
namespace {

constexpr int BK = 64;

// ------------------------------------------------------------- V packing
// Slot of a key inside its 16-key group in a packed V^T row: slots 8*h + e
// (h = lane / 32, e = 0..7) hold key 8*(e/4) + 4*h + e%4, the key that
// register 8*hk + e of an S^T accumulator holds for that lane.
__device__ __forceinline__ int packed_key(int slot) {
  const int g = slot >> 4, h = (slot >> 3) & 1, e = slot & 7;
  return 16 * g + 8 * (e >> 2) + 4 * h + (e & 3);
}

// vt[bh][j][d][slot] = V[bh][64*j + packed_key(slot)][d], zero past N.
// grid (n_k, B*H), 256 threads; one 64-key block per workgroup.
template <int D>
__global__ __launch_bounds__(256) void vt_pack_kernel(const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ vt, int N,
                                                      int n_k) {
  __shared__ uint16_t tile[BK][D + 2];  // +2: odd 32-bit word pitch, conflict-free columns
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const uint16_t* src = v + ((size_t)bh * N + (size_t)j * BK) * D;
  constexpr int CPR = D / 8;
  for (int c = t; c < BK * CPR; c += 256) {
    const int row = c / CPR, ch = c % CPR;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (j * BK + row < N) w = *reinterpret_cast<const uint4*>(src + (size_t)row * D + ch * 8);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[row][ch * 8 + 2 * e] = (uint16_t)(ws[e] & 0xFFFFu);
      tile[row][ch * 8 + 2 * e + 1] = (uint16_t)(ws[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = vt + ((size_t)bh * n_k + j) * (size_t)D * BK;
  for (int c = t; c < D * (BK / 8); c += 256) {  // output chunk: row d, slots 8*g8..+8
    const int d = c / (BK / 8), g8 = c % (BK / 8);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[packed_key(8 * g8 + 2 * e)][d] |
             ((uint32_t)tile[packed_key(8 * g8 + 2 * e + 1)][d] << 16);
    *reinterpret_cast<uint4*>(dst + (size_t)d * BK + 8 * g8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ------------------------------------------------------------ LDS tiles
// K tile: [64 keys][D] row-major; V tile: packed V^T, [D][64 slots]. The
// 16-byte chunks of every row are XOR-swizzled with the row index so that
// the MFMA operand reads (32 rows at one chunk) hit distinct banks: chunk c
// of row r is stored at chunk c ^ (r mod chunks-per-row).
template <int D>
struct Tile {
  static constexpr int KROWB = D * 2;   // bytes per K row
  static constexpr int KCPR = D / 8;    // 16-byte chunks per K row
  static constexpr int VROWB = BK * 2;  // bytes per V^T row (128)
  static constexpr int VCPR = BK / 8;   // 8
  static constexpr int BYTES = BK * D * 2;  // one K or V tile
  static constexpr int STAGE = 2 * BYTES;   // K + V
  __device__ static constexpr int kchunk(int row, int chunk) { return chunk ^ (row & (KCPR - 1)); }
  __device__ static constexpr int vchunk(int row, int chunk) { return chunk ^ (row & (VCPR - 1)); }
};

__device__ __forceinline__ bf16x8 lds_read16(const unsigned char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 16-byte global -> LDS copy without a register round trip (global_load_lds
// dwordx4). `lds` must be the same for the whole wave: lane i's 16 bytes land
// at lds + 16 * i. (Kept out of the kernel templates: the host pass drops a
// template kernel's launch stub when its body names this builtin.)
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const floatx16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[base + e];
  return r;
}

// max / sum over the two half-waves (lane l and lane l ^ 32): the swap
// returns both values of the pair in its two results
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A row's running maximum is only raised (and O rescaled) when a block
// raises it by more than 2^8 in the exponent; until then P <= 2^8, which
// float32 sums and bf16 products carry without loss of relative precision.
constexpr float kRescaleLog2 = 8.0f;

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, (D == 128 && BQ == 64) ? 1 : 2) void sparse_attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ o, int N, int n_q,
    int n_k, int total, float c) {
  constexpr int NW = BQ / 32;               // waves, 32 query rows each
  using T = Tile<D>;
  constexpr int LOADS = BK * D / 8 / 64 / NW;  // 16-byte DMA loads per lane per tile
  constexpr int DT = D / 32;                // O^T tiles per wave
  constexpr int KSTEPS = D / 16;            // k-steps of the QK product

  __shared__ __align__(16) unsigned char smem[2 * T::STAGE];

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;

  // ---- Q fragments (B operand of S^T = K Q^T): query row, 8 d-values
  const int qrow = qi * BQ + wave * 32 + l32;
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = q + head + (size_t)min(qrow, N - 1) * D + 8 * h2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  const int count = min(max(kv_cnt[tile], 0), n_k);
  const int32_t* ids = kv_idx + (size_t)tile * n_k;
  const uint16_t* kh = k + head;
  const uint16_t* vth = vt + (size_t)bh * n_k * D * BK;

  // ---- DMA staging: wave w, load u fills LDS chunks [64*(u*NW+w), +64),
  // lane-linear; each lane fetches the global chunk that the swizzle maps
  // there (the swizzles are involutions). Offsets are loop invariant.
  int krow[LOADS], ksrc[LOADS], vsrc[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int p = 64 * (u * NW + wave) + lane;   // LDS chunk index
    const int kr = p / T::KCPR, vr = p / T::VCPR;
    krow[u] = kr;
    ksrc[u] = kr * D + T::kchunk(kr, p % T::KCPR) * 8;
    vsrc[u] = vr * BK + T::vchunk(vr, p % T::VCPR) * 8;
  }
  auto stage = [&](int j, int buf) {
    unsigned char* kb = smem + buf * T::STAGE;
    unsigned char* vb = kb + T::BYTES;
    const int key0 = j * BK;
    const uint16_t* kt = kh + (size_t)key0 * D;
    const uint16_t* vtt = vth + (size_t)j * D * BK;
    const bool full = key0 + BK <= N;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int dst = 1024 * (u * NW + wave);
      // short last block: K rows past N repeat row N-1 (their scores are
      // masked); packed V is zero there
      const int shift = full ? 0 : max(key0 + krow[u] - (N - 1), 0) * D;
      dma16(kt + ksrc[u] - shift, kb + dst);
      dma16(vtt + vsrc[u], vb + dst);
    }
  };

  // ---- per-lane LDS read offsets (loop invariant)
  int koff[KSTEPS];  // K rows l32 (+32 tau), chunk 2s + h2
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = l32 * T::KROWB + (T::kchunk(l32, 2 * s + h2) << 4);
  int voff[4];       // V^T rows l32 (+32 i), chunk 2G + h2 (slots 16G + 8h2 .. +8)
#pragma unroll
  for (int g = 0; g < 4; ++g) voff[g] = l32 * T::VROWB + (T::vchunk(l32, 2 * g + h2) << 4);

  floatx16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;

  if (count > 0) stage(min(max(ids[0], 0), n_k - 1), 0);

  for (int it = 0; it < count; ++it) {
    const int buf = it & 1;
    const int j = min(max(ids[it], 0), n_k - 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's DMA for buf landed
    __syncthreads();                     // every lane's DMA landed; buf^1 is free
    if (it + 1 < count) stage(min(max(ids[it + 1], 0), n_k - 1), buf ^ 1);
    const unsigned char* kb = smem + buf * T::STAGE;
    const unsigned char* vb = kb + T::BYTES;

    // ---- S^T = K_j Q^T : two 32-key tiles
    floatx16 st[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[tau][r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const bf16x8 a = lds_read16(kb + tau * 32 * T::KROWB + koff[s]);
        st[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[tau], 0, 0, 0);
      }
    }

    // ---- keys past N in a short last block get -inf
    const int nvalid = N - j * BK;
    if (nvalid < BK) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * tau + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (key >= nvalid) st[tau][r] = -INFINITY;
        }
    }

    // ---- online softmax (one query per lane; the two halves hold disjoint keys)
    float mloc = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, st[tau][r]);
    mloc = pair_max(mloc);
    if (__any((mloc - m) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m, mloc);
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    const float mc = m * c;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(st[tau][r], c, -mc));
        st[tau][r] = pr;
        lsum += pr;
      }

    // ---- O^T += V_j^T P^T : 4 k-steps of 16 keys
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        const int G = 2 * tau + hk;
        const bf16x8 pb = pack_bf16x8(st[tau], 8 * hk);
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const bf16x8 a = lds_read16(vb + i * 32 * T::VROWB + voff[G]);
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[i], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O = O^T / l, bf16, rows < N only
  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (qrow < N) {
    uint16_t* orow = o + head + (size_t)qrow * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * i + 8 * g + 4 * h2;
        uint2 pk;
        pk.x = f32_to_bf16_rne(oacc[i][4 * g] * inv) |
               (f32_to_bf16_rne(oacc[i][4 * g + 1] * inv) << 16);
        pk.y = f32_to_bf16_rne(oacc[i][4 * g + 2] * inv) |
               (f32_to_bf16_rne(oacc[i][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
  }
}

template <int D, int BQ>
hipError_t launch_sparse(const AttnLaunch& a, hipStream_t s) {
  const int total = a.B * a.H * a.n_q;
  const float c = a.scale * 1.4426950408889634f;  // scale * log2(e)
  hipLaunchKernelGGL((vt_pack_kernel<D>), dim3(a.n_k, a.B * a.H), dim3(256), 0, s, a.v, a.vt,
                     a.N, a.n_k);
  hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ>), dim3(total), dim3(BQ * 2), 0, s, a.q,
                     a.k, a.vt, a.idx, a.cnt, a.o, a.N, a.n_q, a.n_k, total, c);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int B, int H, int N, int d) {
  const size_t n_k = (N + BK - 1) / BK;
  return (size_t)B * H * n_k * BK * d * sizeof(uint16_t);
}

hipError_t launch_attn(const AttnLaunch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_sparse<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_sparse<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_sparse<64, 128>(a, s);
  return launch_sparse<64, 64>(a, s);
}

}  // namespace sparge
