// Bandwidth-bound element-wise kernels of the Muon step: momentum
// accumulation and the decoupled weight-decay update.
//
// Both stream their operands once (momentum: 12 bytes per element; update:
// 4 + 2 + ... bytes per element depending on dtypes) with 16-byte
// non-temporal vector accesses, one vector per thread and no reuse, so they
// are bound by HBM.
// The arithmetic (momentum_op, update_op) is separate float operations with FP
// contraction switched off: momentum must equal float32 multiply-then-add bit
// for bit.

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

constexpr int kThreads = 256;

__host__ int grid_for(int64_t work_items) {
  // One work item per thread (the loop then runs once): measured on MI355X,
  // a grid that covers the whole array streams about 20 % faster than a
  // grid-stride loop over a few thousand blocks (6.5 vs 5.1-5.4 TB/s for
  // the momentum).  The loop only covers arrays beyond the grid limit.
  int64_t blocks = (work_items + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) blocks = 0x7fffffff;
  if (blocks < 1) blocks = 1;
  return static_cast<int>(blocks);
}

__global__ __launch_bounds__(kThreads) void momentum_vec4_kernel(f32x4* __restrict__ M,
                                                                const f32x4* __restrict__ G,
                                                                int64_t n4, float mu) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += stride) {
    f32x4 m = __builtin_nontemporal_load(&M[i]);
    f32x4 g = __builtin_nontemporal_load(&G[i]);
    m.x = momentum_op(m.x, g.x, mu);
    m.y = momentum_op(m.y, g.y, mu);
    m.z = momentum_op(m.z, g.z, mu);
    m.w = momentum_op(m.w, g.w, mu);
    __builtin_nontemporal_store(m, &M[i]);
  }
}

__global__ __launch_bounds__(kThreads) void momentum_scalar_kernel(float* __restrict__ M,
                                                                  const float* __restrict__ G,
                                                                  int64_t n, float mu) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride)
    M[i] = momentum_op(M[i], G[i], mu);
}

__device__ __forceinline__ void load8_f32(const float* p, float (&v)[8]) {
  f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8_bf16(const uint16_t* p, float (&v)[8]) {
  u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}
__device__ __forceinline__ void store8_f32(float* p, const float (&v)[8]) {
  f32x4 a = {v[0], v[1], v[2], v[3]};
  f32x4 b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p) + 1);
}
__device__ __forceinline__ void store8_bf16(uint16_t* p, const float (&v)[8]) {
  u32x4 a = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
             pack_bf16x2(v[6], v[7])};
  __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(p));
}

template <bool W_BF16, bool O_BF16>
__global__ __launch_bounds__(kThreads) void update_vec8_kernel(void* __restrict__ Wv,
                                                              const void* __restrict__ Ov, int64_t n8,
                                                              float lr, float wd) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n8; i += stride) {
    float w[8], o[8];
    if constexpr (W_BF16) load8_bf16(static_cast<const uint16_t*>(Wv) + i * 8, w);
    else load8_f32(static_cast<const float*>(Wv) + i * 8, w);
    if constexpr (O_BF16) load8_bf16(static_cast<const uint16_t*>(Ov) + i * 8, o);
    else load8_f32(static_cast<const float*>(Ov) + i * 8, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = update_op(w[e], o[e], lr, wd);
    if constexpr (W_BF16) store8_bf16(static_cast<uint16_t*>(Wv) + i * 8, w);
    else store8_f32(static_cast<float*>(Wv) + i * 8, w);
  }
}

template <bool W_BF16, bool O_BF16>
__global__ __launch_bounds__(kThreads) void update_scalar_kernel(void* __restrict__ Wv,
                                                                const void* __restrict__ Ov,
                                                                int64_t begin, int64_t n, float lr,
                                                                float wd) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = begin + static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += stride) {
    float w = W_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(Wv)[i])
                     : static_cast<const float*>(Wv)[i];
    float o = O_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(Ov)[i])
                     : static_cast<const float*>(Ov)[i];
    float r = update_op(w, o, lr, wd);
    if (W_BF16) static_cast<uint16_t*>(Wv)[i] = f32_to_bf16(r);
    else static_cast<float*>(Wv)[i] = r;
  }
}

template <bool W_BF16, bool O_BF16>
hipError_t update_dispatch(void* W, const void* O, int64_t numel, float lr, float wd,
                           hipStream_t stream) {
  const size_t wbytes = W_BF16 ? 2 : 4, obytes = O_BF16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(W) % (8 * wbytes) == 0) &&
                       (reinterpret_cast<uintptr_t>(O) % (8 * obytes) == 0);
  int64_t done = 0;
  if (aligned && numel >= 8) {
    const int64_t n8 = numel / 8;
    hipLaunchKernelGGL((update_vec8_kernel<W_BF16, O_BF16>), dim3(grid_for(n8)), dim3(kThreads), 0,
                       stream, W, O, n8, lr, wd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    done = n8 * 8;
  }
  if (done < numel) {
    hipLaunchKernelGGL((update_scalar_kernel<W_BF16, O_BF16>), dim3(grid_for(numel - done)),
                       dim3(kThreads), 0, stream, W, O, done, numel, lr, wd);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_momentum(float* M, const float* G, int64_t numel, float mu, hipStream_t stream) {
  const bool aligned = (reinterpret_cast<uintptr_t>(M) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(G) % 16 == 0);
  int64_t done = 0;
  if (aligned && numel >= 4) {
    const int64_t n4 = numel / 4;
    hipLaunchKernelGGL(momentum_vec4_kernel, dim3(grid_for(n4)), dim3(kThreads), 0, stream,
                       reinterpret_cast<f32x4*>(M), reinterpret_cast<const f32x4*>(G), n4, mu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    done = n4 * 4;
  }
  if (done < numel) {
    const int64_t rest = numel - done;
    hipLaunchKernelGGL(momentum_scalar_kernel, dim3(grid_for(rest)), dim3(kThreads), 0, stream,
                       M + done, G + done, rest, mu);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_update(void* W, bool w_bf16, const void* O, bool o_bf16, int64_t numel, float lr,
                         float weight_decay, hipStream_t stream) {
  if (w_bf16 && o_bf16) return update_dispatch<true, true>(W, O, numel, lr, weight_decay, stream);
  if (w_bf16) return update_dispatch<true, false>(W, O, numel, lr, weight_decay, stream);
  if (o_bf16) return update_dispatch<false, true>(W, O, numel, lr, weight_decay, stream);
  return update_dispatch<false, false>(W, O, numel, lr, weight_decay, stream);
}

}  // namespace mc
