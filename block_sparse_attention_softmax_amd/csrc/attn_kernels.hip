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
// second product unchanged; V is pre-packed once per call (pack_kernel)
// into key-contiguous tiles in the key order those registers imply, so both
// MFMA A operands are plain 16-byte LDS reads.
//
// K_j and packed V_j tiles are copied global -> LDS by direct-to-LDS loads
// (no register round trip), double-buffered so the copies overlap the
// products of earlier blocks.
#include "internal.h"
#include "tiles.h"
#include "linear_common.h"

#include <type_traits>

namespace sparge {
namespace {

// A row's running maximum is only raised (and O rescaled) when a block
// raises it by more than 2^8 in the exponent; until then P <= 2^8, which
// float32 sums and bf16 products carry without loss of relative precision.
constexpr float kRescaleLog2 = 8.0f;

// ------------------------------------------------------ attention kernel
// Software-pipelined over the listed blocks: the S^T product of block it+1
// is issued while the softmax and the P V product of block it run, so the
// matrix cores have independent work during the softmax. K tiles and packed
// V^T tiles are double-buffered separately, one block apart: during step
// `it` K buffer (it+1)&1 holds K of block it+1 and V buffer it&1 holds V^T
// of block it; the copies issued during step `it` (K of block it+2, V^T of
// block it+1) fill the buffers that step it-1 finished with. They are
// spread one per k-step over the S^T product instead of issued together,
// so the waves of a CU do not queue behind each other's copies.
//
// LIN adds the linear branch over the dropped blocks in the epilogue: O_l =
// phi(Q) H_D / (phi(Q) . z_D) for each wave's 32 queries, with H_D^T (two bf16
// planes, staged in LDS) and z_D of the query block from linear_hd_kernel
// (three-term split-bf16 product: hi hi + hi lo + lo hi, about 16 significant
// bits per operand); the output is O = O_s + alpha[h] O_l, or in the SLA2 mix
// (SLA2 page, section 2A) O = alpha[h][c] O_s + (1 - alpha[h][c]) O_l with the
// scale 1 / (phi(Q) . z_D). Heads whose branch is dropped (lin_on = 0) keep
// O_s (times alpha[h][c] in the mix). LSE also stores every row's log-sum-exp
// of its kept scores, ln(sum_u exp(scale q.k_u)) of the sparse part, for the
// backward.
template <int D, int BQ, bool LIN, bool LSE = false>
__global__ __launch_bounds__(BQ * 2, (D == 128 && BQ == 64) ? 1 : 2) void sparse_attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ o, int H, int N, int n_q,
    int n_k, int total, float c, const float* __restrict__ alpha,
    const uint16_t* __restrict__ hd, const float* __restrict__ zd,
    const int32_t* __restrict__ lin_on, int lin_mode, float* __restrict__ lse) {
  constexpr int NW = BQ / 32;
  using T = Tile<D>;
  constexpr int LOADS = BK * D / 8 / 64 / NW;
  constexpr int DT = D / 32;
  constexpr int KSTEPS = D / 16;

  // K0 K1 V0 V1; buffer b of block i is (i + ...) & 1 as below
  __shared__ __align__(16) unsigned char smem[4 * T::BYTES];
  unsigned char* const kbuf = smem;
  unsigned char* const vbuf = smem + 2 * T::BYTES;

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / n_q, qi = tile % n_q;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;

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
  const size_t vtile = (size_t)D * BK;
  const uint16_t* vth = vt + (size_t)bh * n_k * vtile;
  // the list is read through two 64-entry windows held one entry per lane
  // (entries w0 .. w0+127), so the block loop issues no scalar memory loads
  auto load_win = [&](int base) { return base + lane < n_k ? ids[base + lane] : 0; };
  int w0 = 0;
  int win0 = load_win(0), win1 = load_win(64);
  auto jat = [&](int i) {  // i in [w0, w0 + 128)
    const int r = i - w0;
    const int a = __builtin_amdgcn_readlane(win0, r & 63);
    const int b = __builtin_amdgcn_readlane(win1, r & 63);
    return min(max(r < 64 ? a : b, 0), n_k - 1);
  };

  constexpr int KROWS_U = 64 * NW / T::KCPR, VROWS_U = 64 * NW / T::VCPR;
  constexpr bool KCONST = KROWS_U % T::KCPR == 0, VCONST = VROWS_U % (2 * T::VCPR) == 0;
  uint32_t kbyte[KCONST ? 1 : LOADS], vbyte[VCONST ? 1 : LOADS];
#pragma unroll
  for (int u = 0; u < (KCONST ? 1 : LOADS); ++u) {
    const int p = 64 * (u * NW + wave) + lane;
    const int kr = p / T::KCPR;
    kbyte[u] = (uint32_t)(kr * D + T::kchunk(kr, p % T::KCPR) * 8) * 2u;
  }
#pragma unroll
  for (int u = 0; u < (VCONST ? 1 : LOADS); ++u) {
    const int p = 64 * (u * NW + wave) + lane;
    const int vr = p / T::VCPR;
    vbyte[u] = (uint32_t)(vr * BK + T::vchunk(vr, p % T::VCPR) * 8) * 2u;
  }
  auto kofs = [&](int u) { return KCONST ? kbyte[0] + (uint32_t)(u * KROWS_U * D * 2) : kbyte[u]; };
  auto vofs = [&](int u) { return VCONST ? vbyte[0] + (uint32_t)(u * VROWS_U * BK * 2) : vbyte[u]; };
  auto stageK = [&](int j, int b) {
    unsigned char* kb = kbuf + b * T::BYTES;
    const int key0 = j * BK;
    const char* kt = reinterpret_cast<const char*>(kh + (size_t)key0 * D);
    if (key0 + BK <= N) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) dma16(kt + kofs(u), kb + 1024 * (u * NW + wave));
    } else {  // short last block: K rows past N repeat row N-1 (their scores are masked)
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int krow = (64 * (u * NW + wave) + lane) / T::KCPR;
        const uint32_t shift = (uint32_t)max(key0 + krow - (N - 1), 0) * D * 2u;
        dma16(kt + (kofs(u) - shift), kb + 1024 * (u * NW + wave));
      }
    }
  };
  auto stageV = [&](int j, int b) {  // V^T tile
    const char* vtt = reinterpret_cast<const char*>(vth + (size_t)j * vtile);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) dma16(vtt + vofs(u), vbuf + b * T::BYTES + 1024 * (u * NW + wave));
  };
  int koff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = l32 * T::KROWB + (T::kchunk(l32, 2 * s + h2) << 4);
  int voff[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) voff[g] = l32 * T::VROWB + (T::vchunk(l32, 2 * g + h2) << 4);

  // k-steps [S0, S1) of S^T = K Q^T from the K tile at kb
  auto qk = [&](const unsigned char* kb, floatx16(&st)[2], auto s0_tag, auto s1_tag, auto&& hook) {
    constexpr int S0 = decltype(s0_tag)::value, S1 = decltype(s1_tag)::value;
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
  using Zero = std::integral_constant<int, 0>;
  using Half = std::integral_constant<int, KSTEPS / 2>;
  using Full = std::integral_constant<int, KSTEPS>;

  floatx16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;
  floatx16 sc[2], sn[2];  // S^T of the current and the next block (roles swap each step)
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[tau][r] = 0.0f;
  int jcur = 0;

  if (count > 0) {
    jcur = jat(0);
    stageK(jcur, 0);
    stageV(jcur, 0);
    if (count > 1) stageK(jat(1), 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    qk(kbuf, sc, Zero{}, Full{}, [](int) {});
  }
  // one listed block: softmax and P V of block `it` (S^T in sc), and with
  // NEXT the S^T of block it+1 into sn, interleaved
  auto step = [&](int it, auto next_tag, floatx16(&sc)[2], floatx16(&sn)[2]) {
    constexpr bool NEXT = decltype(next_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K of it+1 and V^T of it landed
    __syncthreads();                     // and every wave is done with step it-1's buffers
    int jn = jcur;
    // copies for later steps, spread one per k-step over the S^T product of
    // block it+1: K of block it+2 (a repeat of it+1 when there is none; that
    // buffer is not read again) and V^T of block it+1
    const char* ksrc = nullptr;
    const char* vsrc = nullptr;
    uint32_t ko[LOADS];
    if constexpr (NEXT) {
      if (it + 1 == w0 + 64) {  // slide the windows; the load lands with this step's copies
        win0 = win1;
        w0 += 64;
        win1 = load_win(w0 + 64);
      }
      jn = jat(it + 1);
      const int jk = it + 2 < count ? jat(it + 2) : jn;
      const int key0 = jk * BK;
      ksrc = reinterpret_cast<const char*>(kh + (size_t)key0 * D);
      vsrc = reinterpret_cast<const char*>(vth + (size_t)jn * vtile);
      if (key0 + BK <= N) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) ko[u] = kofs(u);
      } else {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          const int krow = (64 * (u * NW + wave) + lane) / T::KCPR;
          ko[u] = kofs(u) - (uint32_t)max(key0 + krow - (N - 1), 0) * D * 2u;
        }
      }
    }
    unsigned char* kdst = kbuf + (it & 1) * T::BYTES;
    unsigned char* vdst = vbuf + ((it + 1) & 1) * T::BYTES;
    constexpr int HALF = KSTEPS / 2;
    auto kdma = [&](int sl) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        if (u * HALF / LOADS == sl) dma16(ksrc + ko[u], kdst + 1024 * (u * NW + wave));
    };
    auto vdma = [&](int sl) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        if (u * HALF / LOADS == sl) dma16(vsrc + vofs(u), vdst + 1024 * (u * NW + wave));
    };
    const unsigned char* kn = kbuf + ((it + 1) & 1) * T::BYTES;
    const unsigned char* vb = vbuf + (it & 1) * T::BYTES;

    const int nvalid = N - jcur * BK;  // keys past N in a short last block get -inf
    if (nvalid < BK) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * tau + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (key >= nvalid) sc[tau][r] = -INFINITY;
        }
    }

#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[tau][r] = 0.0f;
    if constexpr (NEXT) qk(kn, sn, Zero{}, Half{}, kdma);

    float mloc = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sc[tau][r]);
    mloc = pair_max(mloc);
    if (__any((mloc - m) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m, mloc);
      const float alpha_r = __builtin_amdgcn_exp2f((m - m_new) * c);
      m = m_new;
      lsum *= alpha_r;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha_r;
    }

    if constexpr (NEXT) qk(kn, sn, Half{}, Full{}, vdma);
    const float mc = m * c;
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
    if constexpr (NEXT) jcur = jn;
  };
  {  // two steps per iteration, the S^T arrays swapping roles
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

  // ---- epilogue: O = O^T / l, with the linear branch or alpha as above; bf16, rows < N only
  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if constexpr (LSE) {  // sum_u exp(scale s_u) = 2^(m c) * ltot; -inf for an empty row
    if (h2 == 0 && qrow < N)
      lse[(size_t)bh * N + qrow] =
          ltot > 0.0f ? (m * c + log2f(ltot)) * 0.6931471805599453f : -INFINITY;
  }
  // LIN: O_l^T (d x 32 queries) = H_D^T phi(Q)^T for this wave's queries, in
  // the oacc layout, and its scale (alpha[h], or 1 in the mix) / (phi(Q_t) .
  // z_D), zero when D_i is empty (z_D = 0). The two H_D^T planes of the query
  // block are copied into the tile buffers (rows swizzled like K tiles) once
  // every wave is past its last block.
  floatx16 lacc[DT];
  float lin_scale = 0.0f;
  bool lin = false;
  if constexpr (LIN) {
    lin = lin_on[bh % H] != 0;  // the same for the whole workgroup
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) lacc[i][r] = 0.0f;
    if (lin) {
      constexpr int NC = 2 * D * D * 2 / 1024;  // 1 KB copies of both planes
      static_assert(NC % NW == 0 && 2 * D * D * 2 <= 4 * T::BYTES,
                    "the H_D^T planes must fit the tile buffers");
      const size_t qb = (size_t)bh * n_q + qi;
      const char* src = reinterpret_cast<const char*>(hd + qb * 2 * D * D);
      __syncthreads();  // every wave is done with the tile buffers
#pragma unroll
      for (int u = 0; u < NC / NW; ++u) {
        const int ci = u * NW + wave, p = 64 * ci + lane;
        const int pl = p / (D * T::KCPR), b = (p / T::KCPR) % D;
        dma16(src + ((size_t)pl * D * D + (size_t)b * D + T::kchunk(b, p % T::KCPR) * 8) * 2,
              smem + 1024 * ci);
      }
      const float* zq = zd + qb * D;
      float den = 0.0f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const float4 z0 = *reinterpret_cast<const float4*>(zq + 16 * s + 8 * h2);
        const float4 z1 = *reinterpret_cast<const float4*>(zq + 16 * s + 8 * h2 + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) den = fmaf(elu1((float)qf[s][e]), zv[e], den);
      }
      den = pair_sum(den);
      lin_scale = den > 0.0f ? (lin_mode == kLinMix ? 1.0f : alpha[bh % H]) / den : 0.0f;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's plane copies landed
      __syncthreads();                     // and every wave's
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        bf16x8 qhi, qlo;  // phi(Q) in the qf layout, split in two bf16 terms
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float fq = elu1((float)qf[s][e]);
          qhi[e] = (__bf16)fq;
          qlo[e] = (__bf16)(fq - (float)qhi[e]);
        }
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int b = 32 * i + l32;
          const int ofs = b * D * 2 + (T::kchunk(b, 2 * s + h2) << 4);
          const bf16x8 hhi = lds_read16(smem + ofs), hlo = lds_read16(smem + D * D * 2 + ofs);
          lacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hhi, qhi, lacc[i], 0, 0, 0);
          lacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hhi, qlo, lacc[i], 0, 0, 0);
          lacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hlo, qhi, lacc[i], 0, 0, 0);
        }
      }
      __syncthreads();  // every wave is done with the planes before the O tiles reuse the space
    }
  }
  // O leaves through LDS: each wave writes its 32 x D tile into its own slice
  // of buffers no wave reads any more (the K tiles, which the last block does
  // not use, or with LIN the planes' space), rows with their 16-byte chunks
  // XOR-swizzled, then copies whole rows out, so that every store instruction
  // writes 64 x 16 contiguous bytes
  static_assert(NW * 32 * D * 2 <= 2 * T::BYTES, "the O tiles must fit two staging buffers");
  unsigned char* stg = smem + wave * 32 * D * 2;
  store_rows_via_lds<D>(stg, o + head, qi * BQ + wave * 32, N, lane, [&](int i, int g) {
    const int d0 = 32 * i + 8 * g + 4 * h2;
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = oacc[i][4 * g + e] * inv;
    if constexpr (LIN) {
      if (lin_mode == kLinMix) {  // alpha[h][d0 .. d0 + 3]
        const float4 a4 = *reinterpret_cast<const float4*>(alpha + (size_t)(bh % H) * D + d0);
        const float a[4] = {a4.x, a4.y, a4.z, a4.w};
        if (lin) {  // the same for the whole workgroup: one branch, not one per value
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[e] = fmaf(a[e], y[e], (1.0f - a[e]) * (lacc[i][4 * g + e] * lin_scale));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = a[e] * y[e];
        }
      } else if (lin) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(lacc[i][4 * g + e], lin_scale, y[e]);
      }
    }
    uint2 pk;
    pk.x = pack2_bf16(y[0], y[1]);
    pk.y = pack2_bf16(y[2], y[3]);
    return pk;
  });
}

template <int D, int BQ, bool LIN>
hipError_t launch_sparse(const AttnLaunch& a, hipStream_t s, AttnPhase phase) {
  const int total = a.B * a.H * a.n_q;
  const float c = a.scale * 1.4426950408889634f;  // scale * log2(e)
  const int BH = a.B * a.H;
  if (phase != kAttendOnly) {
    if constexpr (LIN)
      hipLaunchKernelGGL(linear_flags_kernel, dim3(1), dim3(kFlagThreads), 0, s, a.alpha,
                         a.lin_mode, D, a.drop_below, a.B, a.H, a.lin_on, a.lin_lists);
    if constexpr (LIN)
      hipLaunchKernelGGL((linear_pack_kernel<D>), dim3(a.n_k, BH), dim3(2 * D), 0, s, a.v, a.k,
                         a.vt, a.hj, a.N, a.n_k, a.lin_on, a.H);
    else
      hipLaunchKernelGGL((pack_kernel<D>), dim3(a.n_k, BH), dim3(2 * D), 0, s, a.v, a.vt, a.N,
                         a.n_k);
  }
  if (phase != kPackOnly) {
    if constexpr (LIN) {
      const int rows = BH * a.n_q, n_kw = (a.n_k + 31) / 32;
      hipLaunchKernelGGL(linear_mdrop_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a.idx, a.cnt,
                         a.mbits, a.n_k, n_kw, rows);
      hipLaunchKernelGGL((linear_hd_kernel<D>),
                         dim3((lin_cols<D>() + 127) / 128, (a.n_q + 255) / 256, BH), dim3(256), 0,
                         s, a.hj, a.mbits, a.hd, a.zd, a.n_q, a.n_k, n_kw, a.lin_on, a.H);
      if (a.lse)
        hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, true, true>), dim3(total), dim3(BQ * 2),
                           0, s, a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total,
                           c, a.alpha, a.hd, a.zd, a.lin_on, a.lin_mode, a.lse);
      else
        hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, true>), dim3(total), dim3(BQ * 2), 0, s,
                           a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total, c,
                           a.alpha, a.hd, a.zd, a.lin_on, a.lin_mode, nullptr);
    } else if (a.lse) {
      hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, false, true>), dim3(total), dim3(BQ * 2),
                         0, s, a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total,
                         c, nullptr, nullptr, nullptr, nullptr, 0, a.lse);
    } else {
      hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, false>), dim3(total), dim3(BQ * 2), 0, s,
                         a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total, c,
                         nullptr, nullptr, nullptr, nullptr, 0, nullptr);
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int B, int H, int N, int d) {
  const size_t n_k = (N + BK - 1) / BK;
  return (size_t)B * H * n_k * BK * d * sizeof(uint16_t);
}

// Linear workspace, in order: packed V^T, the per-key-block
// summaries (two bf16 planes of D*D + D per block), the drop matrix (bf16,
// rows of n_k rounded up to 32), H_D^T planes and z_D per query block, the
// branch flags and head lists; every part 256-byte aligned.
size_t linear_layout(AttnLaunch& a, unsigned char* w, int B, int H, int N, int d, int block_q) {
  const size_t BH = (size_t)B * H, n_k = (N + BK - 1) / BK, n_q = (N + block_q - 1) / block_q;
  const size_t n_kw = (n_k + 31) / 32, cols = (size_t)d * d + d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = w ? w + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  a.vt = reinterpret_cast<uint16_t*>(take(attn_workspace_bytes(B, H, N, d)));
  a.hj = reinterpret_cast<uint16_t*>(take(BH * n_k * 2 * cols * 2));
  a.mbits = reinterpret_cast<uint32_t*>(take(BH * n_q * n_kw * 4));
  a.hd = reinterpret_cast<uint16_t*>(take(BH * n_q * 2 * (size_t)d * d * 2));
  a.zd = reinterpret_cast<float*>(take(BH * n_q * d * 4));
  a.lin_on = reinterpret_cast<int32_t*>(take((size_t)H * 4));
  a.lin_lists = reinterpret_cast<int32_t*>(take((2 + 2 * BH) * 4));
  return off;
}

size_t linear_workspace_bytes(int B, int H, int N, int d, int block_q) {
  AttnLaunch a{};
  return linear_layout(a, nullptr, B, H, N, d, block_q);
}

hipError_t launch_attn(const AttnLaunch& a, hipStream_t s, AttnPhase phase) {
  if (a.alpha) {
    if (a.d == 128) return launch_sparse<128, 128, true>(a, s, phase);
    return launch_sparse<64, 64, true>(a, s, phase);
  }
  if (a.d == 128 && a.block_q == 128) return launch_sparse<128, 128, false>(a, s, phase);
  if (a.d == 128 && a.block_q == 64) return launch_sparse<128, 64, false>(a, s, phase);
  if (a.d == 64 && a.block_q == 128) return launch_sparse<64, 128, false>(a, s, phase);
  return launch_sparse<64, 64, false>(a, s, phase);
}

}  // namespace sparge
