// Tile layouts and small device helpers shared by the attention forward and
// backward translation units: the key-contiguous packing of a [rows][d]
// operand into [d][64 slots] blocks in the key order of an MFMA accumulator,
// the XOR-swizzled LDS tiles, direct-to-LDS copies and bf16 packing.
#pragma once

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

// phi(x) = elu(x) + 1, the feature map of the linear branch: x + 1 above 0,
// else e^x = 2^(x log2 e) by the hardware exp2. Its relative error, about
// |x| 2^-24 from the rounded product plus the instruction's own ulp, lies far
// below the bf16 rounding phi goes through; both sides are computed and one
// selected, so there is no branch per element.
__device__ __forceinline__ float elu1(float x) {
  const float e = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
  return x > 0.0f ? x + 1.0f : e;
}

// vt[bh][j][d][slot] = V[bh][64*j + packed_key(slot)][d], zero past N.
// grid (n_k, B*H), 2*D threads; one 64-key block per workgroup. Thread t
// takes keys 4q..4q+3 (q = t % 16) at d = 8c..8c+7 (c = t / 16): four 16-byte
// rows in, transposed in registers, eight 8-byte pieces out. The four keys
// occupy four consecutive slots, and the 16 lanes sharing c write whole
// 128-byte rows of the packed block.
// F16 stores the values as fp16 instead: a bf16 value converts to fp16
// exactly when its magnitude lies in [2^-14, 65504].
template <int D, bool F16 = false>
__global__ __launch_bounds__(2 * D) void pack_kernel(const uint16_t* __restrict__ v,
                                                     uint16_t* __restrict__ vt, int N, int n_k) {
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int q = t & 15, c = t >> 4;
  // slot of key 4q: group q/4, then the inverse of packed_key within it
  const int slot0 = 16 * (q >> 2) + 8 * (q & 1) + 4 * ((q >> 1) & 1);
  const uint16_t* src = v + ((size_t)bh * N + (size_t)j * BK) * D + c * 8;
  uint32_t x[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = 4 * q + r;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (j * BK + key < N) {
      u = *reinterpret_cast<const uint4*>(src + (size_t)key * D);
      if constexpr (F16) {
        uint32_t* p = &u.x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)bf16_lo(p[e])) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)bf16_hi(p[e])) << 16);
      }
    }
    x[r][0] = u.x; x[r][1] = u.y; x[r][2] = u.z; x[r][3] = u.w;
  }
  uint16_t* dst = vt + ((size_t)bh * n_k + j) * (size_t)D * BK + (size_t)(8 * c) * BK + slot0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {  // d = 8c + 2e (low halves) and 8c + 2e + 1 (high)
    uint2 lo, hi;
    lo.x = (x[0][e] & 0xFFFFu) | (x[1][e] << 16);
    lo.y = (x[2][e] & 0xFFFFu) | (x[3][e] << 16);
    hi.x = (x[0][e] >> 16) | (x[1][e] & 0xFFFF0000u);
    hi.y = (x[2][e] >> 16) | (x[3][e] & 0xFFFF0000u);
    *reinterpret_cast<uint2*>(dst + (size_t)(2 * e) * BK) = lo;
    *reinterpret_cast<uint2*>(dst + (size_t)(2 * e + 1) * BK) = hi;
  }
}

// ------------------------------------------------------------ LDS tiles
// K tile: [64 keys][D] row-major; V tile: packed V^T, [D][64 slots]. The
// 16-byte chunks of every row are XOR-swizzled with the row index so that
// the MFMA operand reads (16 lanes per cycle, 16 consecutive rows at one
// logical chunk) cover all 64 banks: K rows are 256 bytes, so chunk c of row
// r goes to c ^ (r mod 16); V^T rows are 128 bytes, two per bank window, so
// chunk c goes to c ^ ((r / 2) mod 8).
template <int D>
struct Tile {
  static constexpr int KROWB = D * 2;   // bytes per K row
  static constexpr int KCPR = D / 8;    // 16-byte chunks per K row
  static constexpr int VROWB = BK * 2;  // bytes per V^T row (128)
  static constexpr int VCPR = BK / 8;   // 8
  static constexpr int BYTES = BK * D * 2;  // one K, V^T or phi(K)^T tile
  __device__ static constexpr int kchunk(int row, int chunk) { return chunk ^ (row & (KCPR - 1)); }
  __device__ static constexpr int vchunk(int row, int chunk) { return chunk ^ ((row >> 1) & (VCPR - 1)); }
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
// The same for 4 bytes per lane (global_load_lds_dword): lane i's word lands
// at lds + 4 * i.
__device__ __forceinline__ void dma4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// Orders a wave's own LDS writes before its later LDS reads of other lanes'
// data (a wave's LDS instructions execute in order; this keeps the compiler
// from moving the reads up)
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A wave's 32 output rows (queries row0 .. row0+31, D channels, bf16) leave
// through LDS: pk(i, g) gives the 8 bytes of channels 32 i + 8 g + 4 h .. +3
// (h = lane / 32) for the lane's query lane % 32, in the register layout of a
// 32x32 MFMA accumulator. They are written into the wave's own tile at `stg`
// (32 x D, 16-byte chunks XOR-swizzled by row) and copied out as whole rows,
// 64 x 16 contiguous bytes per store instruction, with non-temporal stores
// (the rows are not read again by the kernel). Rows at or past N are skipped.
template <int D, typename F>
__device__ __forceinline__ void store_rows_via_lds(unsigned char* stg, uint16_t* out, int row0,
                                                   int N, int lane, F&& pk) {
  constexpr int CPR = D / 8, DT = D / 32;  // 16-byte chunks per row, 32-channel tiles
  const int l32 = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * i + 8 * g + 4 * h2;
      const int chunk = (d0 >> 3) ^ (l32 & (CPR - 1));
      *reinterpret_cast<uint2*>(stg + l32 * D * 2 + chunk * 16 + (d0 & 4) * 2) = pk(i, g);
    }
  wave_lds_fence();
  constexpr int RPI = 64 / CPR;  // rows per copy instruction
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int rr = r0 + lane / CPR, cc = lane % CPR;
    const uint4 val = *reinterpret_cast<const uint4*>(stg + rr * D * 2 + ((cc ^ (rr & (CPR - 1))) << 4));
    const int row = row0 + rr;
    if (row < N) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 w = {val.x, val.y, val.z, val.w};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out + (size_t)row * D + cc * 8));
    }
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// 32-bit LDS address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(p);
}

// NR transposing LDS reads (ds_read_b64_tr_b16; NR = 8 or 16): within each
// group of 16 lanes, lane i receives element i & 3 of the 4-element rows that
// lanes 4e + (i >> 2), e = 0..3, address. Written as one asm block that also
// waits for them: as a builtin the compiler holds such a read until every
// direct-to-LDS copy in flight has landed, the next stage's included.
template <int NR>
__device__ __forceinline__ void lds_read_tr(v4i16 (&r)[NR], const uint32_t (&a)[NR]) {
  static_assert(NR == 8 || NR == 16, "8 or 16 reads");
  if constexpr (NR == 8) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %18\n\tds_read_b64_tr_b16 %3, %19\n\t"
        "ds_read_b64_tr_b16 %4, %20\n\tds_read_b64_tr_b16 %5, %21\n\t"
        "ds_read_b64_tr_b16 %6, %22\n\tds_read_b64_tr_b16 %7, %23\n\t"
        "ds_read_b64_tr_b16 %8, %24\n\tds_read_b64_tr_b16 %9, %25\n\t"
        "ds_read_b64_tr_b16 %10, %26\n\tds_read_b64_tr_b16 %11, %27\n\t"
        "ds_read_b64_tr_b16 %12, %28\n\tds_read_b64_tr_b16 %13, %29\n\t"
        "ds_read_b64_tr_b16 %14, %30\n\tds_read_b64_tr_b16 %15, %31\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]),
          "v"(a[15])
        : "memory");
  }
}

__device__ __forceinline__ bf16x8 join_tr(v4i16 lo, v4i16 hi) {
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, (v8i16)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup barrier without the memory fence of __syncthreads, whose release
// half waits for every direct-to-LDS copy still in flight, prefetches of later
// stages included. Callers first wait (s_waitcnt vmcnt) for the copies the
// next step reads; every LDS read of a buffer is consumed before the barrier
// after which that buffer is refilled. The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// two floats -> two bf16 (round to nearest even) in one dword, low half first
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const floatx16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[base + e];
  return r;
}

// acc + sum of the 8 bf16 values (v_dot2 against ones, float32 accumulate)
__device__ __forceinline__ float row_sum_bf16x8(const bf16x8& p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 pr = {p[e], p[e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
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

}  // namespace
}  // namespace sparge
