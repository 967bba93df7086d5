// Measurement probes: what this chip sustains for the two resources the
// Muon step is bound by, measured on the box next to the step itself.
//   mfma_probe_kernel  back-to-back v_mfma_f32_32x32x16_bf16 on register
//                      operands (no memory traffic): the sustained dense bf16
//                      matrix rate at the clock the chip actually runs;
//   copy_probe_kernel  a plain device copy in 16-byte accesses: the sustained
//                      HBM bandwidth (bytes read + bytes written).
// The caller times the launches (HIP events on the same stream); the flop and
// byte counts are stated in include/muon.h.
#include "muon_device.h"

namespace muon {

// Each wave keeps kChains independent accumulators, so consecutive MFMAs do
// not wait for each other's results; 8 waves per block (2 per SIMD).
constexpr int kChains = 4;

__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, float* sink) {
  const int tid = threadIdx.x;
  // operands that depend on the lane, so nothing folds at compile time
  const float s = 1.0f + 1e-3f * (float)(tid & 63);
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<bf16_t>(s * (float)(e + 1) * 1e-2f);
    b[e] = static_cast<bf16_t>((float)(8 - e) * 1e-2f);
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float v = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) v += acc[c][r];
  sink[(long long)blockIdx.x * blockDim.x + tid] = v;
}

// Grid-stride copy with four independent 16-byte loads in flight per thread
// before their stores.
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4_t* __restrict__ src,
                                                         u32x4_t* __restrict__ dst, long long n16) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride],
                  v3 = src[i + 3 * stride];
    dst[i] = v0;
    dst[i + stride] = v1;
    dst[i + 2 * stride] = v2;
    dst[i + 3 * stride] = v3;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_mfma_probe(int blocks, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(512), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, long long n16, int blocks,
                             hipStream_t s) {
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
  return hipGetLastError();
}

}  // namespace muon
