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
// LIN adds the linear branch over the dropped blocks with a second set of
// BQ/32 waves in the workgroup (H waves), which pass the attention waves'
// barriers one for one (the attention waves' loop is the plain one). Per
// listed block, H wave w accumulates rows 32w..32w+31 of H_kept +=
// phi(K_j)^T V_j and its share of z_kept += sum phi(K_j), from the V^T tile
// the attention waves staged and a phi(K)^T tile the H waves copy beside it;
// when more than half of the blocks are listed they instead sum the blocks
// not listed (found from a bitmap of the list), copying both tiles of those
// themselves, and H_D is that sum rather than H_tot - H_kept.
// The H waves' matrix products fill the attention waves' softmax gaps on the
// same SIMDs, and the attention waves carry no extra accumulator. At the end
// the H waves form H_D (and z_D likewise) in LDS, then
// O_l = phi(Q) H_D / (phi(Q) . z_D) for the queries of the attention wave of
// the same index (three-term split-bf16 MFMA product, about 16 significant
// bits per operand), and hand O_l and the scale alpha[h] / (phi(Q) . z_D)
// over through LDS in the attention wave's own register layout; the
// attention wave writes O = O_s + alpha[h] * O_l, or in the SLA2 mix (SLA2
// page, section 2A) O = alpha[h][c] O_s + (1 - alpha[h][c]) O_l with the
// scale 1 / (phi(Q) . z_D). Heads whose branch is dropped (lin_on = 0) are
// left to a second launch of the plain kernel, which scales O_s by
// alpha[h][c] in the mix; each launch maps its workgroups onto its own heads
// through the lists of linear_flags_kernel.
//
// SEL (always with LIN) adds the head selection and the alpha scaling of the
// epilogue; the plain kernel without it is compiled without either. LSE
// (plain kernel only) also stores every row's log-sum-exp of its kept scores,
// ln(sum_u exp(scale q.k_u)) of the sparse part, for the backward.
template <int D, int BQ, bool LIN, bool SEL = LIN, bool LSE = false>
__global__ __launch_bounds__(BQ * (LIN ? 4 : 2), (LIN || (D == 128 && BQ == 64)) ? 1 : 2) void sparse_attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ o, int H, int N, int n_q,
    int n_k, int total, float c, const float* __restrict__ alpha,
    const uint16_t* __restrict__ phikt, const float* __restrict__ lin_h,
    const float* __restrict__ lin_z, const int32_t* __restrict__ sel_lists, int lin_mode,
    float* __restrict__ lse) {
  constexpr int NW = BQ / 32;
  using T = Tile<D>;
  constexpr int LOADS = BK * D / 8 / 64 / NW;
  constexpr int DT = D / 32;
  constexpr int KSTEPS = D / 16;
  static_assert(!LIN || NW == DT, "the linear branch needs one wave per 32 rows of d");

  // K0 K1 V0 V1 (LIN: phi(K)^T 0, 1, the H waves' V^T 0, 1 and the kept-block
  // bitmap); buffer b of block i is (i + ...) & 1 as below
  __shared__ __align__(16)
      unsigned char smem[LIN ? 8 * T::BYTES + kMaxLinKeyBlocks / 8 : 4 * T::BYTES];
  unsigned char* const kbuf = smem;
  unsigned char* const vbuf = smem + 2 * T::BYTES;
  unsigned char* const pbuf = smem + 4 * T::BYTES;
  unsigned char* const hvbuf = smem + 6 * T::BYTES;
  uint32_t* const kbits = reinterpret_cast<uint32_t*>(smem + (LIN ? 8 : 4) * T::BYTES);

  // with a head selection, LIN runs the (batch, head) pairs whose linear
  // branch is on and the plain kernel the others: the first n_sel * n_q
  // workgroups take the selected heads' query blocks, spread over the XCDs
  // like the full grid, and the rest exit
  int tile;
  if constexpr (SEL) {
    const int n_sel = sel_lists[LIN ? 0 : 1];
    if ((int)blockIdx.x >= n_sel * n_q) return;
    const int t2 = xcd_remap(blockIdx.x, n_sel * n_q);
    tile = sel_lists[2 + (LIN ? 0 : total / n_q) + t2 / n_q] * n_q + t2 % n_q;
  } else {
    tile = xcd_remap(blockIdx.x, total);
  }
  const int bh = tile / n_q, qi = tile % n_q;
  const int t = threadIdx.x, lane = t & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(t >> 6);
  // LIN: waves NW.. are H waves (H_kept and z_kept for the d rows 32*wave..);
  // the first NW waves run the attention itself and issue every copy
  const bool hwave = LIN && wave_id >= NW;
  const int wave = hwave ? wave_id - NW : wave_id;
  const int h2 = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * N * D;

  const int qrow = qi * BQ + wave * 32 + l32;
  bf16x8 qf[KSTEPS];  // (H waves load the rows of their attention wave, for phi(Q))
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
  const uint16_t* pkh = LIN ? phikt + (size_t)bh * n_k * vtile : nullptr;
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
  auto stageP = [&](int j, int b) {  // phi(K)^T tile (LIN)
    const char* ptt = reinterpret_cast<const char*>(pkh + (size_t)j * vtile);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) dma16(ptt + vofs(u), pbuf + b * T::BYTES + 1024 * (u * NW + wave));
  };

  // LIN: the H waves sum phi(K_j)^T V_j over the listed blocks (H_D = H_tot -
  // that sum, the listed blocks' tiles arriving with the attention's own) or,
  // when that is the longer list, over the blocks not listed (their tiles
  // copied by the H waves themselves). Deciding needs the number of distinct
  // listed blocks: a bitmap of the list, built before the first barrier.
  const bool maybe_off = LIN && count > n_k - count && n_k <= kMaxLinKeyBlocks;
  const int words = (n_k + 31) / 32;
  if constexpr (LIN) {
    if (maybe_off) {  // bits past n_k count as listed
      for (int w = t; w < words; w += BQ * 4)
        kbits[w] = 32 * w + 32 > n_k ? ~((1u << (n_k - 32 * w)) - 1u) : 0u;
      __syncthreads();
      for (int e = t; e < count; e += BQ * 4) {
        const int j = min(max(ids[e], 0), n_k - 1);
        atomicOr(&kbits[j >> 5], 1u << (j & 31));
      }
    }
  }

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
  // H waves accumulate H_kept (rows 32*wave..) in oacc and their share of
  // z_kept (entry 32*wave + l32, split over the half-waves) in lsum
  floatx16 sc[2], sn[2];  // S^T of the current and the next block (roles swap each step)
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[tau][r] = 0.0f;
  int jcur = 0;

  if (count > 0) {
    if (!hwave) {
      jcur = jat(0);
      stageK(jcur, 0);
      stageV(jcur, 0);
      if (count > 1) stageK(jat(1), 1);
    } else if (!maybe_off) {
      stageP(jat(0), 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (!hwave) qk(kbuf, sc, Zero{}, Full{}, [](int) {});
  }
  // hoff: the H waves take the n_off < count blocks not listed (every wave
  // counts the bitmap's clear bits); otherwise the listed blocks, whose first
  // phi(K)^T tile, when the route was open until now, they copy here (read
  // after step 0's barrier)
  int n_off = n_k;
  bool hoff = false;
  if constexpr (LIN) {
    if (maybe_off) {
      int c0 = 0;
      for (int w = lane; w < words; w += 64) c0 += __popc(~kbits[w]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c0 += __shfl_xor(c0, o);
      n_off = __builtin_amdgcn_readfirstlane(c0);
      hoff = n_off < count;
    }
    if (hwave && maybe_off && !hoff) stageP(jat(0), 0);
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
  if (hwave) {
    // H waves: one barrier per listed block, like the attention waves' steps;
    // H += phi(K_j)^T V_j and z += sum phi(K_j) from a (V^T, phi(K)^T) pair
    auto h_block = [&](const unsigned char* vbh, const unsigned char* pbh) {
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const bf16x8 pkf = lds_read16(pbh + wave * 32 * T::VROWB + voff[G]);
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum += (float)pkf[e];
#pragma unroll
        for (int i = 0; i < DT; ++i)
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              pkf, lds_read16(vbh + i * 32 * T::VROWB + voff[G]), oacc[i], 0, 0, 0);
      }
    };
    if (hoff) {
      // the blocks not listed, in increasing order: block e is copied (phi(K)^T
      // to phi buffer e & 1, V^T to the H waves' V buffer e & 1) after barrier
      // e and summed after barrier e + 1, so n_off < count barriers suffice
      auto next_off = [&](int j) {  // the first block after j that is not listed
        int w = (j + 1) >> 5;
        uint32_t m = w < words ? ~kbits[w] & (~0u << ((j + 1) & 31)) : 0u;
        while (m == 0u && ++w < words) m = ~kbits[w];
        return m ? 32 * w + __builtin_ctz(m) : n_k;
      };
      int jo = next_off(-1);
      for (int it = 0; it < count; ++it) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (it < n_off) {
          const char* ptt = reinterpret_cast<const char*>(pkh + (size_t)jo * vtile);
          const char* vtt = reinterpret_cast<const char*>(vth + (size_t)jo * vtile);
#pragma unroll
          for (int u = 0; u < LOADS; ++u) {
            dma16(ptt + vofs(u), pbuf + (it & 1) * T::BYTES + 1024 * (u * NW + wave));
            dma16(vtt + vofs(u), hvbuf + (it & 1) * T::BYTES + 1024 * (u * NW + wave));
          }
          jo = next_off(jo);
        }
        if (it >= 1 && it - 1 < n_off)
          h_block(hvbuf + ((it - 1) & 1) * T::BYTES, pbuf + ((it - 1) & 1) * T::BYTES);
      }
    } else {
      // the listed blocks: V^T of block it from the attention waves' buffer
      // it & 1, its phi(K)^T (copied by the H waves after the barrier before)
      // from phi buffer it & 1; list entries come from the lane-held windows,
      // slid like the attention waves' (no scalar loads next to LDS reads)
      for (int it = 0; it < count; ++it) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (it + 1 < count) {
          if (it + 1 == w0 + 64) {
            win0 = win1;
            w0 += 64;
            win1 = load_win(w0 + 64);
          }
          stageP(jat(it + 1), (it + 1) & 1);
        }
        h_block(vbuf + (it & 1) * T::BYTES, pbuf + (it & 1) * T::BYTES);
      }
    }
  } else {
    int it = 0;
    if constexpr (LIN) {  // (two steps per iteration need more registers than LIN has left)
      for (; it + 1 < count; ++it) {
        step(it, std::true_type{}, sc, sn);
        sc[0] = sn[0];
        sc[1] = sn[1];
      }
      if (count > 0) step(it, std::false_type{}, sc, sn);
    } else {  // two steps per iteration, the S^T arrays swapping roles
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
  }

  // ---- epilogue: O = O^T / l, with the linear branch or alpha as above; bf16, rows < N only
  const float ltot = pair_sum(lsum);  // (H waves: their z entry 32*wave + l32)
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if constexpr (LSE) {  // sum_u exp(scale s_u) = 2^(m c) * ltot; -inf for an empty row
    if (!hwave && h2 == 0 && qrow < N)
      lse[(size_t)bh * N + qrow] =
          ltot > 0.0f ? (m * c + log2f(ltot)) * 0.6931471805599453f : -INFINITY;
  }
  // LIN: O_l for this lane's (d, query) entries, in the oacc layout, and
  // alpha[h] / (phi(Q_t) . z_D) for its query, handed over through LDS by the
  // H wave of the same index
  const float4* yl = nullptr;
  const float* ys = nullptr;
  if constexpr (LIN) {
    // the staging buffers become H_D^T [D][D+4] fp32 and z_D [D], then the
    // per-lane O_l fragments [NW][DT*4][64 lanes] float4 and scales [NW][64]
    constexpr int HP = D + 4;
    float* ht = reinterpret_cast<float*>(smem);
    float* zd = ht + D * HP;
    static_assert(D * HP * 4 + D * 4 <= 6 * T::BYTES, "H_D must fit the staging buffers");
    static_assert(NW * DT * 4 * 64 * 16 + NW * 64 * 4 <= 6 * T::BYTES,
                  "O_l must fit the staging buffers");
    float4* ylds = reinterpret_cast<float4*>(smem);
    float* ysds = reinterpret_cast<float*>(ylds + NW * DT * 4 * 64);
    const bool dropped = count < n_k;  // D_i is empty when every block is kept
    __syncthreads();                   // every wave is done with the staging buffers
    if (dropped && hwave) {  // H_D = H_tot - the listed sum, or the sum itself
      const float* Ht = lin_h + (size_t)bh * D * D;
      if (hoff) {
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(ht + (32 * i + l32) * HP + 32 * wave + 8 * g + 4 * h2) =
                make_float4(oacc[i][4 * g + 0], oacc[i][4 * g + 1], oacc[i][4 * g + 2],
                            oacc[i][4 * g + 3]);
        if (h2 == 0) zd[32 * wave + l32] = ltot;
      } else {
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int a0 = 32 * wave + 8 * g + 4 * h2, b = 32 * i + l32;
            float4 x;
            x.x = Ht[(size_t)(a0 + 0) * D + b] - oacc[i][4 * g + 0];
            x.y = Ht[(size_t)(a0 + 1) * D + b] - oacc[i][4 * g + 1];
            x.z = Ht[(size_t)(a0 + 2) * D + b] - oacc[i][4 * g + 2];
            x.w = Ht[(size_t)(a0 + 3) * D + b] - oacc[i][4 * g + 3];
            *reinterpret_cast<float4*>(ht + b * HP + a0) = x;
          }
        if (h2 == 0) zd[32 * wave + l32] = lin_z[(size_t)bh * D + 32 * wave + l32] - ltot;
      }
    }
    __syncthreads();
    float lin_scale = 0.0f;  // alpha[h] / (phi(Q_t) . z_D)
    if (dropped && hwave) {
      // O_l^T (d x 32 queries) = H_D^T phi(Q)^T; phi(Q) in the qf layout
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
      float den = 0.0f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        bf16x8 qhi, qlo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float fq = elu1((float)qf[s][e]);
          den = fmaf(fq, zd[16 * s + 8 * h2 + e], den);
          qhi[e] = (__bf16)fq;
          qlo[e] = (__bf16)(fq - (float)qhi[e]);
        }
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const float* hp = ht + (32 * i + l32) * HP + 16 * s + 8 * h2;
          const float4 h0 = *reinterpret_cast<const float4*>(hp);
          const float4 h1 = *reinterpret_cast<const float4*>(hp + 4);
          const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          bf16x8 hhi, hlo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hhi[e] = (__bf16)hv[e];
            hlo[e] = (__bf16)(hv[e] - (float)hhi[e]);
          }
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hhi, qhi, oacc[i], 0, 0, 0);
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hhi, qlo, oacc[i], 0, 0, 0);
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hlo, qhi, oacc[i], 0, 0, 0);
        }
      }
      den = pair_sum(den);
      lin_scale = den > 0.0f ? (lin_mode == kLinMix ? 1.0f : alpha[bh % H]) / den : 0.0f;
    }
    __syncthreads();  // every H wave is done reading H_D^T
    if (dropped && hwave) {
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          ylds[((wave * DT + i) * 4 + g) * 64 + lane] =
              make_float4(oacc[i][4 * g + 0], oacc[i][4 * g + 1], oacc[i][4 * g + 2],
                          oacc[i][4 * g + 3]);
      ysds[wave * 64 + lane] = lin_scale;
    }
    __syncthreads();
    if (dropped) {
      yl = ylds;
      ys = ysds;
    }
  }
  // O leaves through LDS: each wave writes its 32 x D tile into its own slice
  // of buffers no wave reads any more (the K tiles, which the last block does
  // not use; LIN: the H waves' V^T tiles, past the H_D and O_l staging), rows
  // with their 16-byte chunks XOR-swizzled, then copies whole rows out, so
  // that every store instruction writes 64 x 16 contiguous bytes
  if (!hwave) {
    static_assert(NW * 32 * D * 2 <= 2 * T::BYTES, "the O tiles must fit two staging buffers");
    unsigned char* stg = smem + (LIN ? 6 * T::BYTES : 0) + wave * 32 * D * 2;
    store_rows_via_lds<D>(stg, o + head, qi * BQ + wave * 32, N, lane, [&](int i, int g) {
      const int d0 = 32 * i + 8 * g + 4 * h2;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = oacc[i][4 * g + e] * inv;
      // mix: alpha[h][d0..d0+3] (plain kernel: the scale of a dropped branch's alpha O_s)
      const bool mix = SEL && (LIN ? lin_mode == kLinMix : alpha != nullptr);
      float a[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if (mix) {
        const float4 a4 = *reinterpret_cast<const float4*>(alpha + (size_t)(bh % H) * D + d0);
        a[0] = a4.x; a[1] = a4.y; a[2] = a4.z; a[3] = a4.w;
      }
      bool have_l = false;
      float lv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sl = 0.0f;
      if constexpr (LIN) {
        if (yl) {
          const float4 l = yl[((wave * DT + i) * 4 + g) * 64 + lane];
          lv[0] = l.x; lv[1] = l.y; lv[2] = l.z; lv[3] = l.w;
          sl = ys[wave * 64 + lane];
          have_l = true;
        }
      }
      if (mix) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = have_l ? fmaf(a[e], y[e], (1.0f - a[e]) * (lv[e] * sl)) : a[e] * y[e];
      } else if (have_l) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(lv[e], sl, y[e]);
      }
      uint2 pk;
      pk.x = pack2_bf16(y[0], y[1]);
      pk.y = pack2_bf16(y[2], y[3]);
      return pk;
    });
  }
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
    hipLaunchKernelGGL((pack_kernel<D, LIN>), dim3(a.n_k, BH), dim3(2 * D), 0, s, a.v, a.k,
                       a.vt, a.phikt, a.N, a.n_k, a.lin_on, a.H);
    if constexpr (LIN) {
      hipLaunchKernelGGL((linear_total_kernel<D>), dim3(kLinSplit, BH), dim3(D * 2), 0, s,
                         a.phikt, a.vt, a.part_h, a.part_z, a.n_k, a.lin_on, a.H);
      hipLaunchKernelGGL((linear_reduce_kernel<D>), dim3(BH, (D * D + D + 255) / 256), dim3(256),
                         0, s, a.part_h, a.part_z, a.lin_h, a.lin_z, a.lin_on, a.H);
    }
  }
  if (phase != kPackOnly) {
    if constexpr (LIN) {
      // heads whose branch is on, then (plain kernel, times alpha in the mix) the others
      const float* mix_alpha = a.lin_mode == kLinMix ? a.alpha : nullptr;
      if (a.lse) {
        hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, true, true, true>), dim3(total),
                           dim3(BQ * 4), 0, s, a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q,
                           a.n_k, total, c, a.alpha, a.phikt, a.lin_h, a.lin_z, a.lin_lists,
                           a.lin_mode, a.lse);
        hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, false, true, true>), dim3(total),
                           dim3(BQ * 2), 0, s, a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q,
                           a.n_k, total, c, mix_alpha, nullptr, nullptr, nullptr, a.lin_lists,
                           a.lin_mode, a.lse);
      } else {
        hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, true>), dim3(total), dim3(BQ * 4), 0, s,
                           a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total, c,
                           a.alpha, a.phikt, a.lin_h, a.lin_z, a.lin_lists, a.lin_mode, nullptr);
        hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, false, true>), dim3(total), dim3(BQ * 2),
                           0, s, a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total,
                           c, mix_alpha, nullptr, nullptr, nullptr, a.lin_lists, a.lin_mode,
                           nullptr);
      }
    } else if (a.lse) {
      hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, false, false, true>), dim3(total),
                         dim3(BQ * 2), 0, s, a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q,
                         a.n_k, total, c, nullptr, nullptr, nullptr, nullptr, nullptr, 0, a.lse);
    } else {
      hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BQ, false>), dim3(total), dim3(BQ * 2), 0, s,
                         a.q, a.k, a.vt, a.idx, a.cnt, a.o, a.H, a.N, a.n_q, a.n_k, total, c,
                         nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr);
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int B, int H, int N, int d) {
  const size_t n_k = (N + BK - 1) / BK;
  return (size_t)B * H * n_k * BK * d * sizeof(uint16_t);
}

size_t linear_workspace_bytes(int B, int H, int N, int d) {
  const size_t BH = (size_t)B * H;
  return 2 * attn_workspace_bytes(B, H, N, d) +                // packed V, packed phi(K)
         BH * ((size_t)d * d + d) * (1 + kLinSplit) * sizeof(float) +  // totals + partials
         ((size_t)H + 2 + 2 * BH) * sizeof(int32_t);  // branch flags and head lists
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
