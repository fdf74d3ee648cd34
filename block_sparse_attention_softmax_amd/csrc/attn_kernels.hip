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
// second product unchanged: the key order they imply inside each 16-key step
// is matched by the order in which V^T is laid out in LDS.
//
// K_j and V_j are staged in LDS, double-buffered: the global loads of block
// j+1 are issued before the products of block j and written to the other
// buffer at the top of the next iteration, so one barrier per block suffices.
#include "internal.h"

namespace sparge {
namespace {

constexpr int BK = 64;

template <int D>
struct Lds {
  static constexpr int KS = D * 2 + 16;  // K row pitch (bytes), 16 B pad
  static constexpr int VS = BK * 2 + 16; // V^T row pitch (bytes), 16 B pad
  static constexpr int KBUF = BK * KS;
  static constexpr int VBUF = D * VS;
  static constexpr int STAGE = KBUF + VBUF;
};

__device__ __forceinline__ bf16x8 lds_read16(const unsigned char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const floatx16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[base + e];
  return r;
}

// Slot (in bf16 units, within a 64-key row of V^T) of the first of the four
// consecutive keys 4*kg .. 4*kg+3. Inside each group of 16 keys, slots
// 8*h + e (h = lane / 32, e = 0..7) hold key 8*(e/4) + 4*h + e%4, which is
// the key that register 8*hk + e of the S^T accumulator holds for that lane.
__device__ __forceinline__ int vt_slot(int kg) {
  const int m = kg & 3;
  return 16 * (kg >> 2) + 8 * (m & 1) + 4 * (m >> 1);
}

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, (D == 128 && BQ == 64) ? 1 : 2) void sparse_attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ o, int N, int n_q,
    int n_k, int total, float c) {
  constexpr int NT = BQ * 2;               // threads (BQ/32 waves)
  constexpr int KCH = D / 8;               // 16-byte chunks per row
  constexpr int KUNITS = BK * KCH;         // K chunks per block
  constexpr int KPT = KUNITS / NT;         // K chunks per thread
  constexpr int VUNITS = 16 * KCH;         // (4 keys x 8 d) V units per block
  constexpr int VPT = (VUNITS + NT - 1) / NT;
  constexpr int DT = D / 32;               // O^T tiles per wave
  constexpr int KSTEPS = D / 16;           // k-steps of the QK product
  using L = Lds<D>;
  static_assert(KUNITS % NT == 0, "K staging must divide evenly");

  __shared__ __align__(16) unsigned char smem[2 * L::STAGE];

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;

  // ---- Q fragments (B operand of S^T = K Q^T): query row, 8 d-values
  const int qrow = qi * BQ + wave * 32 + l32;
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = q + head + (size_t)qrow * D + 8 * h2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (qrow < N) {
        qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)0.0f;
      }
    }
  }

  const int count = min(max(kv_cnt[tile], 0), n_k);
  const int32_t* ids = kv_idx + (size_t)tile * n_k;
  const uint16_t* kh = k + head;
  const uint16_t* vh = v + head;

  uint4 kreg[KPT];
  uint4 vreg[VPT][4];

  auto gload = [&](int j) {
    const int key0 = j * BK;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int cu = t + NT * u, row = cu / KCH, ch = cu % KCH;
      const int key = key0 + row;
      kreg[u] = key < N ? *reinterpret_cast<const uint4*>(kh + (size_t)key * D + ch * 8)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int vu = t + NT * u;
      if (vu < VUNITS) {
        const int kg = vu & 15, ch = vu >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 4 * kg + r;
          vreg[u][r] = key < N
                           ? *reinterpret_cast<const uint4*>(vh + (size_t)key * D + ch * 8)
                           : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto swrite = [&](int buf) {
    unsigned char* ks = smem + buf * L::STAGE;
    unsigned char* vt = ks + L::KBUF;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int cu = t + NT * u, row = cu / KCH, ch = cu % KCH;
      *reinterpret_cast<uint4*>(ks + row * L::KS + ch * 16) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int vu = t + NT * u;
      if (vu < VUNITS) {
        const int kg = vu & 15, ch = vu >> 4;
        unsigned char* dst = vt + (ch * 8) * L::VS + vt_slot(kg) * 2;
        const uint32_t w0[4] = {vreg[u][0].x, vreg[u][0].y, vreg[u][0].z, vreg[u][0].w};
        const uint32_t w1[4] = {vreg[u][1].x, vreg[u][1].y, vreg[u][1].z, vreg[u][1].w};
        const uint32_t w2[4] = {vreg[u][2].x, vreg[u][2].y, vreg[u][2].z, vreg[u][2].w};
        const uint32_t w3[4] = {vreg[u][3].x, vreg[u][3].y, vreg[u][3].z, vreg[u][3].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // d = 8*ch + 2w (low halves) and 8*ch + 2w + 1 (high halves)
          uint2 lo, hi;
          lo.x = (w0[w] & 0xFFFFu) | (w1[w] << 16);
          lo.y = (w2[w] & 0xFFFFu) | (w3[w] << 16);
          hi.x = (w0[w] >> 16) | (w1[w] & 0xFFFF0000u);
          hi.y = (w2[w] >> 16) | (w3[w] & 0xFFFF0000u);
          *reinterpret_cast<uint2*>(dst + (2 * w) * L::VS) = lo;
          *reinterpret_cast<uint2*>(dst + (2 * w + 1) * L::VS) = hi;
        }
      }
    }
  };

  floatx16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;

  int jcur = count > 0 ? min(max(ids[0], 0), n_k - 1) : 0;
  if (count > 0) gload(jcur);

  for (int it = 0; it < count; ++it) {
    const int buf = it & 1;
    swrite(buf);
    __syncthreads();
    const int j = jcur;
    if (it + 1 < count) {
      jcur = min(max(ids[it + 1], 0), n_k - 1);
      gload(jcur);
    }
    const unsigned char* ks = smem + buf * L::STAGE;
    const unsigned char* vt = ks + L::KBUF;

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
        const bf16x8 a = lds_read16(ks + (32 * tau + l32) * L::KS + (16 * s + 8 * h2) * 2);
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

    // ---- online softmax (one query per lane; halves hold disjoint keys)
    float mloc = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, st[tau][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m, mloc);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    m = m_new;
    const float mc = m_new * c;
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
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
        const bf16x8 pb = pack_bf16x8(st[tau], 8 * hk);
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const bf16x8 a =
              lds_read16(vt + (32 * i + l32) * L::VS + (32 * tau + 16 * hk + 8 * h2) * 2);
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[i], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O = O^T / l, bf16, rows < N only
  const float ltot = lsum + __shfl_xor(lsum, 32);
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
  hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ>), dim3(total), dim3(BQ * 2), 0, s, a.q,
                     a.k, a.v, a.idx, a.cnt, a.o, a.N, a.n_q, a.n_k, total, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnLaunch& a, hipStream_t s) {
  if (a.d == 128 && a.block_q == 128) return launch_sparse<128, 128>(a, s);
  if (a.d == 128 && a.block_q == 64) return launch_sparse<128, 64>(a, s);
  if (a.d == 64 && a.block_q == 128) return launch_sparse<64, 128>(a, s);
  return launch_sparse<64, 64>(a, s);
}

}  // namespace sparge
