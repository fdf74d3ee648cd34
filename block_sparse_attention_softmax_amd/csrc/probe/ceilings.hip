// Measurement probe (not part of the attention path): the dense bf16 MFMA
// throughput this GPU sustains, as the denominator beside the 2.5 PFLOP/s
// nameplate. Every wave keeps four independent 32x32 accumulators busy with
// v_mfma_f32_32x32x16_bf16 on register operands (CHAINS independent
// accumulators per wave), so nothing but the matrix cores (and the clock they
// run at) limits the rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

namespace {

template <int kChains>
__global__ __launch_bounds__(256, 2) void mfma_bf16_probe_kernel(float* __restrict__ out,
                                                                 int iters, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(e - (int)threadIdx.x));
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the products live
}

}  // namespace

extern "C" {

// FLOPs one launch performs with `blocks` workgroups of 256 threads.
double sparge_probe_mfma_flops(int blocks, int iters, int chains) {
  return (double)blocks * 4 /* waves */ * iters * chains * (2.0 * 32 * 32 * 16);
}

// Launches the probe with 4 or 8 chains per wave on `stream` (hipStream_t as
// void*); `out` holds blocks*256 floats. Returns 0, or a HIP error code.
int sparge_probe_mfma_bf16(float* out, int blocks, int iters, int chains, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (chains != 4 && chains != 8))
    return (int)hipErrorInvalidValue;
  if (chains == 4)
    hipLaunchKernelGGL(mfma_bf16_probe_kernel<4>, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out, iters, 1.0f / 1024.0f);
  else
    hipLaunchKernelGGL(mfma_bf16_probe_kernel<8>, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out, iters, 1.0f / 1024.0f);
  return (int)hipGetLastError();
}

}  // extern "C"
