// Per-head max logit, S_max^h = (1/sqrt(d)) max_{b,i,j} Q[b,h,i] . K[b,h,j],
// with the logit matrix never written anywhere ("Kimi K2 内部机制", MuonClip
// section, core maths: max over the batch and over all token pairs).
//
// bf16 path (d in {64, 128, 192}, d_c and d_r multiples of 8):
//   A 512-thread workgroup (8 wave64s) owns 512 query rows of one (b, h); each
//   wave keeps its 64 rows of Q as MFMA fragments in registers for the whole
//   kernel and streams every key row of (b, h) through a double-buffered LDS
//   stage of 64 keys x d.  Per key block a wave issues 2 x 2 x (d/16)
//   v_mfma_f32_32x32x16_bf16 and folds the 64 x 64 float32 logits into a
//   16-register running max.  The key row is assembled in LDS from the
//   head's own part Kc[b,h,j] and the shared rotary part Kr[b,j] (MLA).
//   Consecutive workgroups of one (b, h) are kept on one XCD so the key
//   stream is read from that XCD's L2.
// float32 path (any other shape, either dtype): a plain LDS-tiled FMA kernel.
//
// Both finish with a workgroup max and one atomic max per workgroup into
// smax[h] (float max through integer atomics; exact and order-independent).
// NaN logits are skipped by the IEEE maxNum of v_max_f32; a head without a
// numeric logit keeps the -inf written by the initialising kernel.

#include <math.h>

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

// Float atomic max through integer atomics: for x >= 0 the int order of the
// bits is the float order; for x < 0 the unsigned order is reversed.
__device__ __forceinline__ void atomic_max_float(float* addr, float x) {
  if (x != x) return;
  if (__float_as_int(x) >= 0) atomicMax(reinterpret_cast<int*>(addr), __float_as_int(x));
  else atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(x));
}

__global__ void init_kernel(float* smax, int64_t H) {
  const int64_t h = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (h < H) smax[h] = -INFINITY;
}

// ------------------------------------------------------------------ bf16 MFMA
constexpr int kMfmaThreads = 512;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerBlock = kRowsPerWave * (kMfmaThreads / 64);  // 512
constexpr int kKeys = 64;                                          // key rows per LDS stage

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D>
__global__ __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void maxlogit_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                          const uint16_t* __restrict__ Kr, int H, int Sq, int Sk, int d_c,
                          int blocks_per_bh, float* __restrict__ smax, float scale) {
  constexpr int kUnits = D / 8;   // 16-byte units per key row
  constexpr int kSteps = D / 16;  // MFMA k-steps
  constexpr int kStageUnits = kKeys * kUnits;
  constexpr int kLoadsPerThread = (kStageUnits + kMfmaThreads - 1) / kMfmaThreads;
  __shared__ u32x4 ks[2][kKeys][kUnits];
  __shared__ float red[kMfmaThreads / 64];

  const uint32_t bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = bid / blocks_per_bh;
  const int ib = bid % blocks_per_bh;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int d_r = D - d_c, uc = d_c / 8;

  const uint16_t* Qbh = Q + (static_cast<int64_t>(b) * H + h) * Sq * D;
  const uint16_t* Kcbh = Kc + (static_cast<int64_t>(b) * H + h) * Sk * d_c;
  const uint16_t* Krb = Kr ? Kr + static_cast<int64_t>(b) * Sk * d_r : nullptr;

  // ---- this wave's 64 query rows as MFMA "A" fragments (row = lane % 32)
  const int row_base = ib * kRowsPerBlock + wave * kRowsPerWave;
  bf16x8 qf[2][kSteps];
  bool row_ok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = row_base + t * 32 + frag_row;
    row_ok[t] = i < Sq;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok[t]) v = *reinterpret_cast<const u32x4*>(Qbh + static_cast<int64_t>(i) * D + 16 * s + 8 * frag_half);
      qf[t][s] = as_bf16x8(v);
    }
  }
  // Rows this lane's accumulator registers cover (for masking the row tail):
  // register r of tile t is row 8*(r/4) + 4*frag_half + r%4 of that 32-row tile.
  const bool any_row_tail = row_base + kRowsPerWave > Sq;

  // ---- key staging: unit u of key row r goes to ks[s][r][u ^ (r & 7)]
  u32x4 stage[kLoadsPerThread];
  auto load_keys = [&](int j0) {
#pragma unroll
    for (int l = 0; l < kLoadsPerThread; ++l) {
      const int idx = tid + l * kMfmaThreads;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (idx < kStageUnits) {
        const int r = idx / kUnits, u = idx % kUnits, j = j0 + r;
        if (j < Sk) {
          if (u < uc) v = *reinterpret_cast<const u32x4*>(Kcbh + static_cast<int64_t>(j) * d_c + 8 * u);
          else v = *reinterpret_cast<const u32x4*>(Krb + static_cast<int64_t>(j) * d_r + 8 * (u - uc));
        }
      }
      stage[l] = v;
    }
  };
  auto store_keys = [&](int s) {
#pragma unroll
    for (int l = 0; l < kLoadsPerThread; ++l) {
      const int idx = tid + l * kMfmaThreads;
      if (idx < kStageUnits) {
        const int r = idx / kUnits, u = idx % kUnits;
        ks[s][r][u ^ (r & 7)] = stage[l];
      }
    }
  };

  f32x16 run;
#pragma unroll
  for (int r = 0; r < 16; ++r) run[r] = -INFINITY;

  const int NJ = (Sk + kKeys - 1) / kKeys;
  load_keys(0);
  store_keys(0);
  __syncthreads();
  for (int jb = 0; jb < NJ; ++jb) {
    const int cur = jb & 1;
    if (jb + 1 < NJ) load_keys((jb + 1) * kKeys);

    f32x16 acc[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[t][u] = f32x16{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int unit = (2 * s + frag_half) ^ (lane & 7);
      bf16x8 kf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) kf[u] = as_bf16x8(ks[cur][u * 32 + frag_row][unit]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[u], acc[t][u], 0, 0, 0);
    }

    // mask the tails: key column j = jb*64 + u*32 + lane%32; query rows per register
    const bool key_tail = (jb + 1) * kKeys > Sk;
    if (key_tail || any_row_tail) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bool col_ok = jb * kKeys + u * 32 + frag_row < Sk;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = row_base + t * 32 + 8 * (r >> 2) + 4 * frag_half + (r & 3);
            if (!col_ok || i >= Sq) acc[t][u][r] = -INFINITY;
          }
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      run[r] = fmaxf(fmaxf(run[r], fmaxf(acc[0][0][r], acc[0][1][r])), fmaxf(acc[1][0][r], acc[1][1][r]));

    if (jb + 1 < NJ) store_keys(cur ^ 1);
    __syncthreads();
  }

  // ---- workgroup max, one atomic per workgroup
  float m = run[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, run[r]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) {
    float w = red[0];
    for (int i = 1; i < kMfmaThreads / 64; ++i) w = fmaxf(w, red[i]);
    if (w != -INFINITY) atomic_max_float(&smax[h], w * scale);
  }
}

// ------------------------------------------------------------------ generic
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

template <int D>
hipError_t launch_mfma(const void* Q, const void* Kc, const void* Kr, int64_t B, int64_t H, int64_t Sq,
                       int64_t Sk, int64_t d_c, float* smax, float scale, hipStream_t stream) {
  const int64_t blocks_per_bh = (Sq + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = blocks_per_bh * B * H;
  hipLaunchKernelGGL((maxlogit_mfma_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(kMfmaThreads),
                     0, stream, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(Kc),
                     static_cast<const uint16_t*>(Kr), static_cast<int>(H), static_cast<int>(Sq),
                     static_cast<int>(Sk), static_cast<int>(d_c), static_cast<int>(blocks_per_bh), smax,
                     scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_maxlogit_init(float* smax, int64_t H, hipStream_t stream) {
  hipLaunchKernelGGL(init_kernel, dim3(static_cast<unsigned>((H + 255) / 256)), dim3(256), 0, stream,
                     smax, H);
  return hipGetLastError();
}

hipError_t launch_maxlogit(const void* Q, const void* Kc, const void* Kr, bool bf16, int64_t B,
                           int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                           hipStream_t stream) {
  const int64_t d = d_c + d_r;
  const float scale = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
  const bool aligned16 = (reinterpret_cast<uintptr_t>(Q) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(Kc) % 16 == 0) &&
                         (Kr == nullptr || reinterpret_cast<uintptr_t>(Kr) % 16 == 0);
  const bool mfma_ok = bf16 && aligned16 && d_c % 8 == 0 && d_r % 8 == 0 &&
                       (d == 64 || d == 128 || d == 192) && Sq <= INT32_MAX &&
                       Sk <= INT32_MAX && B * H * ((Sq + kRowsPerBlock - 1) / kRowsPerBlock) <= INT32_MAX;
  if (mfma_ok) {
    switch (d) {
      case 64: return launch_mfma<64>(Q, Kc, Kr, B, H, Sq, Sk, d_c, smax, scale, stream);
      case 128: return launch_mfma<128>(Q, Kc, Kr, B, H, Sq, Sk, d_c, smax, scale, stream);
      default: return launch_mfma<192>(Q, Kc, Kr, B, H, Sq, Sk, d_c, smax, scale, stream);
    }
  }
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
