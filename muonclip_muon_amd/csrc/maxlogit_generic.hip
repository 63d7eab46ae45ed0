// Per-head max logit for the shapes the bf16 MFMA kernel does not cover
// (float32 inputs, other head dims, fewer than 64 keys, unaligned pointers):
// S_max^h = (1/sqrt(d)) max_{b,i,j} Q[b,h,i] . K[b,h,j] ("Kimi K2 内部机制",
// MuonClip section, core maths), with K = [Kc || shared Kr] (MLA) or Kc (MHA).
// A plain LDS-tiled float32 FMA kernel: each 256-thread workgroup owns 64
// query rows of one (b, h) and walks all keys in 64 x 64 logit tiles, 4 x 4
// per thread, staging 32-wide head-dim slices of Q and K in LDS.  The
// logits stay in registers; a workgroup max then one atomic max per
// workgroup into smax[h].
//
// This file keeps IEEE NaN semantics (unlike the MFMA kernel's file, which is
// built without them): fmaxf skips a NaN logit (IEEE maxNum), so a head
// whose logits are all NaN keeps the -inf written by init_kernel.

#include <math.h>

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

__global__ void init_kernel(float* smax, int64_t H) {
  const int64_t h = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (h < H) smax[h] = -INFINITY;
}

constexpr int kGenThreads = 256;
constexpr int kGenTile = 64;  // 64 x 64 logits per iteration, 4 x 4 per thread
constexpr int kGenDk = 32;    // head-dim slice staged in LDS

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// grid (ceil(Sq/64), H, B)
template <bool BF16>
__global__ __launch_bounds__(kGenThreads) void maxlogit_generic_kernel(
    const void* __restrict__ Q, const void* __restrict__ Kc, const void* __restrict__ Kr, int64_t H,
    int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* __restrict__ smax, float scale) {
  __shared__ float qs[kGenTile][kGenDk + 1];
  __shared__ float kt[kGenTile][kGenDk + 1];
  __shared__ float red[kGenThreads / 64];
  const int64_t b = blockIdx.z, h = blockIdx.y, i0 = static_cast<int64_t>(blockIdx.x) * kGenTile;
  const int64_t d = d_c + d_r;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int64_t qbase = (b * H + h) * Sq * d;
  const int64_t kcbase = (b * H + h) * Sk * d_c;
  const int64_t krbase = b * Sk * d_r;
  float m = -INFINITY;
  for (int64_t j0 = 0; j0 < Sk; j0 += kGenTile) {
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < d; k0 += kGenDk) {
      for (int e = tid; e < kGenTile * kGenDk; e += kGenThreads) {
        const int r = e / kGenDk, c = e % kGenDk;
        const int64_t i = i0 + r, j = j0 + r, k = k0 + c;
        qs[r][c] = (i < Sq && k < d) ? ld_elem<BF16>(Q, qbase + i * d + k) : 0.f;
        float kv = 0.f;
        if (j < Sk && k < d) kv = k < d_c ? ld_elem<BF16>(Kc, kcbase + j * d_c + k)
                                          : ld_elem<BF16>(Kr, krbase + j * d_r + (k - d_c));
        kt[r][c] = kv;
      }
      __syncthreads();
#pragma unroll 4
      for (int c = 0; c < kGenDk; ++c) {
        float qv[4], kv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) qv[a] = qs[ty + 16 * a][c];
#pragma unroll
        for (int a = 0; a < 4; ++a) kv[a] = kt[tx + 16 * a][c];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a][e] = fmaf(qv[a], kv[e], acc[a][e]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + ty + 16 * a < Sq && j0 + tx + 16 * e < Sk) m = fmaxf(m, acc[a][e]);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float w = red[0];
    for (int i = 1; i < kGenThreads / 64; ++i) w = fmaxf(w, red[i]);
    if (w != -INFINITY) atomic_max_float(&smax[h], w * scale);
  }
}


}  // namespace

hipError_t launch_maxlogit_init(float* smax, int64_t H, hipStream_t stream) {
  hipLaunchKernelGGL(init_kernel, dim3(static_cast<unsigned>((H + 255) / 256)), dim3(256), 0, stream,
                     smax, H);
  return hipGetLastError();
}

hipError_t launch_maxlogit_generic(const void* Q, const void* Kc, const void* Kr, bool bf16, int64_t B,
                                   int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                                   float scale, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>((Sq + kGenTile - 1) / kGenTile), static_cast<unsigned>(H),
            static_cast<unsigned>(B));
  if (bf16)
    hipLaunchKernelGGL(maxlogit_generic_kernel<true>, grid, dim3(kGenThreads), 0, stream, Q, Kc, Kr, H,
                       Sq, Sk, d_c, d_r, smax, scale);
  else
    hipLaunchKernelGGL(maxlogit_generic_kernel<false>, grid, dim3(kGenThreads), 0, stream, Q, Kc, Kr,
                       H, Sq, Sk, d_c, d_r, smax, scale);
  return hipGetLastError();
}

}  // namespace mc
