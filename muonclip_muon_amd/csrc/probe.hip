// Measurement aids (not part of the optimizer step): the two self-measured
// ceilings the step's kernels are compared against on the same GPU.
//
//  * mfma_probe_kernel: every wave issues independent
//    v_mfma_f32_32x32x16_bf16 back to back on register operands (16
//    accumulator tiles, 256 AGPRs), no memory traffic in the loop.  Its rate
//    is the MFMA ceiling at the clock the chip actually holds under full
//    matrix load; with random operands the multiplier inputs toggle as they
//    do in a real GEMM, with zero operands the chip draws less power and
//    clocks higher.
//  * copy_probe_kernel: a plain 16-byte-per-lane copy, one vector per thread, the
//    self-measured HBM stream rate that the element-wise kernels are compared
//    against (each byte read once and written once).

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

constexpr int kProbeThreads = 256;

// 32-bit mix (the finaliser of MurmurHash3), for operand bits only.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// A bf16 operand with a random sign and mantissa and an exponent near 1, so
// the accumulators stay finite for any iteration count used here.
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) {
  const uint32_t lo = 0x3f00u | (h & 0x807fu);
  const uint32_t hi = 0x3f00u | ((h >> 16) & 0x807fu);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_probe_kernel(int64_t iters, int zero_operands, float* __restrict__ out) {
  const uint32_t tid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 va, vb;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      va[w] = zero_operands ? 0u : rand_bf16x2(mix32(tid * 64u + i * 8u + w));
      vb[w] = zero_operands ? 0u : rand_bf16x2(mix32(tid * 64u + i * 8u + 4u + w + 0x9e3779b9u));
    }
    a[i] = __builtin_bit_cast(bf16x8, va);
    b[i] = __builtin_bit_cast(bf16x8, vb);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[x][y][r];
  out[tid] = s;
}

__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_mfma_probe(int64_t workgroups, int64_t iters, bool zero_operands, float* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kProbeThreads), 0, stream,
                     iters, zero_operands ? 1 : 0, out);
  return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  // one vector per thread (a grid that covers the array streams faster than
  // a grid-stride loop over a few thousand blocks); the loop only covers
  // arrays beyond the grid limit
  int64_t blocks = (n16 + kProbeThreads - 1) / kProbeThreads;
  if (blocks > 0x7fffffff) blocks = 0x7fffffff;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace mc
