// Newton-Schulz input stage: the workspace geometry, the pre-scale and the
// norm.
//
//   pre-scale  X_0 = M_b, or M_b^T when rows > cols, unscaled, as a bf16
//              matrix of high parts and an int8 matrix coding the low parts
//              (x - high; about 16 significant bits together, mc_device.h),
//              written into the zero-padded
//              n_pad x m_pad workspace layout the GEMMs use, plus float32
//              partial sums of squares per 4096-
//              element block; one block per matrix then combines them in
//              double in a fixed order (deterministic), giving
//              inv_b = 1 / (||M_b||_F + eps), which the first Newton-Schulz
//              step's GEMM epilogues apply.  In the fused step the same pass
//              first does M_b <- mu M_b + G_b in place.
// The pre-scale moves 8-element runs (16-byte vectors where the row length
// and the alignment allow); the transposing variant goes through a 64 x 64
// LDS tile so both the read and the write side are coalesced.  The output
// O = out_scale * X (or X^T) is written by the last step's GEMM epilogue.

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {

namespace {
constexpr int kThreads = 256;
// One block covers 8192 elements (one norm partial each): the tiled kernel
// 64 rows x 128 columns, the row-strip kernel 32 rows x 256 columns.
constexpr int kBlockElems = 8192;
constexpr int kTR = 64, kTC = 128;    // tile of the tiled (transposing) kernel
constexpr int kSR = 32, kSC = 256;    // strip of the row kernel
}  // namespace

static inline int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }
static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

NsGeometry ns_geometry(int64_t batch, int64_t rows, int64_t cols) {
  NsGeometry g{};
  g.batch = batch;
  g.rows = rows;
  g.cols = cols;
  g.transposed = rows > cols;
  g.n = g.transposed ? cols : rows;
  g.m = g.transposed ? rows : cols;
  g.n_pad = round_up(g.n, kNsTile);
  g.m_pad = round_up(g.m, kNsTile);
  g.prescale_tiles = g.n_pad * g.m_pad / kBlockElems;
  const size_t xb = static_cast<size_t>(batch) * g.n_pad * g.m_pad * 2;
  const size_t xlb = static_cast<size_t>(batch) * g.n_pad * g.m_pad;  // int8 low-part codes
  const size_t ab = static_cast<size_t>(batch) * g.n_pad * g.n_pad * 2;
  size_t off = 0;
  g.off_x0 = off; off = align256(off + xb);
  g.off_x1 = off; off = align256(off + xb);
  g.off_xl0 = off; off = align256(off + xlb);
  g.off_xl1 = off; off = align256(off + xlb);
  g.off_a = off; off = align256(off + ab);
  g.off_b = off; off = align256(off + ab);
  g.off_d = off; off = align256(off + static_cast<size_t>(batch) * g.n_pad * 4);
  const int64_t partials = g.prescale_tiles;
  g.off_partials = off; off = align256(off + static_cast<size_t>(batch * partials) * 4);
  g.off_invnorm = off; off = align256(off + static_cast<size_t>(batch) * 4);
  g.total = off;
  return g;
}

namespace {

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x == 0)
    for (int i = 0; i < kThreads / 64; ++i) s += red[i];
  return s;
}

// 8 values as bf16 high parts and the int8 codes of their low parts
__device__ __forceinline__ void pack_hi_lo8(const float (&x)[8], u32x4& hi, u32x2& lo) {
  hi = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  const uint32_t w[4] = {hi.x, hi.y, hi.z, hi.w};
  int32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = enc_lo(x[e], hi_bits(w[e >> 1], e & 1));
  lo = u32x2{pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7])};
}

// grid (batch): inv_b = 1 / (sqrt(sum of partials) + eps), combined in double
__global__ __launch_bounds__(kThreads) void invnorm_kernel(const float* __restrict__ partials,
                                                          int64_t chunks, float eps,
                                                          float* __restrict__ invnorm) {
  __shared__ double red[kThreads];
  const int64_t b = blockIdx.x;
  double acc = 0.0;
  for (int64_t c = threadIdx.x; c < chunks; c += kThreads) acc += partials[b * chunks + c];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) invnorm[b] = static_cast<float>(1.0 / (sqrt(red[0]) + static_cast<double>(eps)));
}

// One element of M (float32 for SRC 1, bf16 for SRC 2) at idx
template <int SRC>
__device__ __forceinline__ float load1_src(const void* M, int64_t idx) {
  if constexpr (SRC == 2) return bf16_to_f32(static_cast<const uint16_t*>(M)[idx]);
  else return static_cast<const float*>(M)[idx];
}

// One 8-element run of M (and of G for SRC 0), loaded without a branch: the
// caller passes a clamped in-bounds index for runs outside the matrix (and
// zeroes their values), so a thread's loads of several passes are all in
// flight before the first of them is used.
template <int SRC>
struct Run8 {
  f32x4 m0, m1, g0, g1;
};
template <int SRC>
__device__ __forceinline__ void load_run8(const void* M, const float* G, int64_t idx, Run8<SRC>& v) {
  if constexpr (SRC == 2) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(M) + idx));
    v.m0 = f32x4{bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y)};
    v.m1 = f32x4{bf16_lo(a.z), bf16_hi(a.z), bf16_lo(a.w), bf16_hi(a.w)};
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(M) + idx);
    v.m0 = __builtin_nontemporal_load(p);
    v.m1 = __builtin_nontemporal_load(p + 1);
    if constexpr (SRC == 0) {
      const f32x4* q = reinterpret_cast<const f32x4*>(G + idx);
      v.g0 = __builtin_nontemporal_load(q);
      v.g1 = __builtin_nontemporal_load(q + 1);
    }
  }
}
// The new M values of a run (momentum for SRC 0, written back to M at idx
// when `in`), as 8 floats; zeros outside the matrix.
template <int SRC>
__device__ __forceinline__ void apply_run8(Run8<SRC>& v, float* M, int64_t idx, float mu, bool in, float (&x)[8]) {
  if constexpr (SRC == 0) {
    v.m0.x = momentum_op(v.m0.x, v.g0.x, mu);
    v.m0.y = momentum_op(v.m0.y, v.g0.y, mu);
    v.m0.z = momentum_op(v.m0.z, v.g0.z, mu);
    v.m0.w = momentum_op(v.m0.w, v.g0.w, mu);
    v.m1.x = momentum_op(v.m1.x, v.g1.x, mu);
    v.m1.y = momentum_op(v.m1.y, v.g1.y, mu);
    v.m1.z = momentum_op(v.m1.z, v.g1.z, mu);
    v.m1.w = momentum_op(v.m1.w, v.g1.w, mu);
    if (in) {
      f32x4* mp = reinterpret_cast<f32x4*>(M + idx);
      __builtin_nontemporal_store(v.m0, mp);
      __builtin_nontemporal_store(v.m1, mp + 1);
    }
  }
  x[0] = in ? v.m0.x : 0.f; x[1] = in ? v.m0.y : 0.f; x[2] = in ? v.m0.z : 0.f; x[3] = in ? v.m0.w : 0.f;
  x[4] = in ? v.m1.x : 0.f; x[5] = in ? v.m1.y : 0.f; x[6] = in ? v.m1.z : 0.f; x[7] = in ? v.m1.w : 0.f;
}

// Fused momentum and pre-scale (SRC = 0).  M_b, G_b are R x C float32 (rows
// x cols); M_b <- fl32(fl32(mu M_b) + G_b) in place (bit-identical to the
// stand-alone momentum), and the new M_b is written unscaled as a (bf16
// high part, int8 low-part code) pair (high parts into S, codes into SL; R_pad x C_pad; rows <= cols:
// X_0 = M) or transposed (T, TL; C_pad x R_pad; rows > cols: X_0 = M^T),
// zero-padded; the other two pointers are null.
// X_0 is written with non-temporal stores (2.8 GB per 64-matrix call: no
// cache holds it until the first product reads it; 3 % faster for the
// transposed tiles, the same for the row strips).
// Each block reads one 64 x 128 tile in 8-element runs (vector loads when
// VEC; 16 lanes cover 512 contiguous bytes of a float32 row) and writes it
// straight from registers or transposed through LDS (8 lanes per output row,
// 128 contiguous bytes of each part); it also writes the float32 sum of
// squares of its tile's new M values to partials[b * tiles + tile].  SRC = 1
// (float32 M) or 2 (bf16 M): the same without momentum (G unused, M only
// read), the unscaled pre-scale of the stand-alone Newton-Schulz call.
// grid (C_pad / 128, R_pad / 64, batch).
template <bool VEC, int SRC>
__global__ __launch_bounds__(kThreads) void momentum_prescale_kernel(void* __restrict__ Mv,
                                                                    const float* __restrict__ G,
                                                                    int64_t batch_stride, float mu, int64_t R,
                                                                    int64_t C, int64_t R_pad, int64_t C_pad,
                                                                    uint16_t* __restrict__ S,
                                                                    uint16_t* __restrict__ T,
                                                                    uint8_t* __restrict__ SL,
                                                                    uint8_t* __restrict__ TL,
                                                                    float* __restrict__ partials) {
  __shared__ float tile[kTR][kTC + 1];
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.z;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTC, r0 = static_cast<int64_t>(blockIdx.y) * kTR;
  float* mb = static_cast<float*>(Mv) + (SRC == 2 ? 0 : b * batch_stride);
  const void* msrc = SRC == 2 ? static_cast<const void*>(static_cast<const uint16_t*>(Mv) + b * batch_stride)
                              : static_cast<const void*>(mb);
  const float* gb = SRC == 0 ? G + b * batch_stride : nullptr;
  uint16_t* sb = S + static_cast<size_t>(b) * R_pad * C_pad;
  uint16_t* tb = T + static_cast<size_t>(b) * R_pad * C_pad;
  uint8_t* slb = SL + static_cast<size_t>(b) * R_pad * C_pad;
  uint8_t* tlb = TL + static_cast<size_t>(b) * R_pad * C_pad;
  const int q = threadIdx.x & 15;
  float ss = 0.f;
  // VEC (C % 8 == 0): a run is wholly inside or wholly outside the matrix;
  // the four passes' loads are issued before any is used
  Run8<SRC> run[VEC ? 4 : 1];
  int64_t idx[VEC ? 4 : 1];
  bool in[VEC ? 4 : 1];
  if constexpr (VEC) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int64_t r = r0 + pass * 16 + (threadIdx.x >> 4), c = c0 + 8 * q;
      in[pass] = r < R && c < C;
      idx[pass] = (r < R ? r : R - 1) * C + (c < C ? c : C - 8);
      if (MC_GUARD(0, idx[pass] >= 0 && idx[pass] + 8 <= R * C)) load_run8<SRC>(msrc, gb, idx[pass], run[pass]);
      else in[pass] = false;
    }
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int rr = pass * 16 + (threadIdx.x >> 4);
    const int64_t r = r0 + rr, c = c0 + 8 * q;
    float x[8];
    if constexpr (VEC) {
      apply_run8<SRC>(run[pass], mb, idx[pass], mu, in[pass], x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = 0.f;
        if (r < R && c + e < C) {
          if constexpr (SRC != 0) {
            x[e] = load1_src<SRC>(msrc, r * C + c + e);
          } else {
            const float m = momentum_op(mb[r * C + c + e], gb[r * C + c + e], mu);
            mb[r * C + c + e] = m;
            x[e] = m;
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    if (S != nullptr) {
      u32x4 hi;
      u32x2 lo;
      pack_hi_lo8(x, hi, lo);
      if (MC_GUARD(1, r < R_pad && c + 8 <= C_pad)) {
        __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(sb + x_off(r, c, R_pad)));
        __builtin_nontemporal_store(lo, reinterpret_cast<u32x2*>(slb + x_off(r, c, R_pad)));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rr][8 * q + e] = x[e];
    }
  }
  // block_sum's barrier also publishes the tile
  const float tile_ss = block_sum(ss, red);
  if (threadIdx.x == 0) partials[b * gridDim.x * gridDim.y + blockIdx.y * gridDim.x + blockIdx.x] = tile_ss;
  if (S != nullptr) return;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int cc = pass * 32 + (threadIdx.x >> 3);
    const int rq = 8 * (threadIdx.x & 7);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[rq + e][cc];
    u32x4 hi;
    u32x2 lo;
    pack_hi_lo8(v, hi, lo);
    if (MC_GUARD(1, c0 + cc < C_pad && r0 + rq + 8 <= R_pad)) {
      __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(tb + x_off(c0 + cc, r0 + rq, C_pad)));
      __builtin_nontemporal_store(lo, reinterpret_cast<u32x2*>(tlb + x_off(c0 + cc, r0 + rq, C_pad)));
    }
  }
}

// The same for rows <= cols with 16-byte aligned rows (the common case),
// with row strips instead of tiles: a block covers 32 rows x 256 columns,
// so every row segment it reads is 1 KB of M and of G, and it writes the 32
// rows of eight 32-column panels of X_0 (x_off): 2 KB of high parts and 1 KB
// of codes contiguous in each panel.
// grid (C_pad / 256, R_pad / 32, batch); 8192 elements per block, like the
// tiles, so the partial-sum count per matrix is the same.  SRC as in
// momentum_prescale_kernel.
template <int SRC>
__global__ __launch_bounds__(kThreads) void momentum_prescale_rows_kernel(
    void* __restrict__ Mv, const float* __restrict__ G, int64_t batch_stride, float mu, int64_t R, int64_t C,
    int64_t R_pad, int64_t C_pad, uint16_t* __restrict__ X0, uint8_t* __restrict__ X0l,
    float* __restrict__ partials) {
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.z;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + 8 * (threadIdx.x & 31);
  float* mb = static_cast<float*>(Mv) + (SRC == 2 ? 0 : b * batch_stride);
  const void* msrc = SRC == 2 ? static_cast<const void*>(static_cast<const uint16_t*>(Mv) + b * batch_stride)
                              : static_cast<const void*>(mb);
  const float* gb = SRC == 0 ? G + b * batch_stride : nullptr;
  uint16_t* xb = X0 + static_cast<size_t>(b) * R_pad * C_pad;
  uint8_t* xlb = X0l + static_cast<size_t>(b) * R_pad * C_pad;
  float ss = 0.f;
  // C % 8 == 0: a run is wholly inside or outside the matrix
  Run8<SRC> run[4];
  int64_t idx[4];
  bool in[4];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int64_t r = static_cast<int64_t>(blockIdx.y) * kSR + pass * 8 + (threadIdx.x >> 5);
    in[pass] = r < R && c < C;
    idx[pass] = (r < R ? r : R - 1) * C + (c < C ? c : C - 8);
    if (MC_GUARD(0, idx[pass] >= 0 && idx[pass] + 8 <= R * C)) load_run8<SRC>(msrc, gb, idx[pass], run[pass]);
    else in[pass] = false;
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int64_t r = static_cast<int64_t>(blockIdx.y) * kSR + pass * 8 + (threadIdx.x >> 5);
    float x[8];
    apply_run8<SRC>(run[pass], mb, idx[pass], mu, in[pass], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    u32x4 hi;
    u32x2 lo;
    pack_hi_lo8(x, hi, lo);
    if (MC_GUARD(1, r < R_pad && c + 8 <= C_pad)) {
      __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(xb + x_off(r, c, R_pad)));
      __builtin_nontemporal_store(lo, reinterpret_cast<u32x2*>(xlb + x_off(r, c, R_pad)));
    }
  }
  const float block_ss = block_sum(ss, red);
  if (threadIdx.x == 0) partials[b * gridDim.x * gridDim.y + blockIdx.y * gridDim.x + blockIdx.x] = block_ss;
}

// SRC 0: momentum (M float32, G); 1 / 2: float32 / bf16 M alone
template <int SRC>
hipError_t launch_prescale_unscaled(void* M, const float* G, int64_t batch_stride, float mu, const NsGeometry& g,
                                    float eps, char* ws, hipStream_t stream) {
  float* partials = reinterpret_cast<float*>(ws + g.off_partials);
  float* invnorm = reinterpret_cast<float*>(ws + g.off_invnorm);
  uint16_t* X0 = reinterpret_cast<uint16_t*>(ws + g.off_x0);
  uint8_t* X0l = reinterpret_cast<uint8_t*>(ws + g.off_xl0);
  const int64_t R = g.rows, C = g.cols;
  const int64_t R_pad = g.transposed ? g.m_pad : g.n_pad, C_pad = g.transposed ? g.n_pad : g.m_pad;
  uint16_t* S = g.transposed ? nullptr : X0;
  uint16_t* T = g.transposed ? X0 : nullptr;
  uint8_t* SL = g.transposed ? nullptr : X0l;
  uint8_t* TL = g.transposed ? X0l : nullptr;
  const size_t align = SRC == 2 ? 16 : 32;  // one 8-element run
  const bool vec = C % 8 == 0 && (g.batch == 1 || batch_stride % 8 == 0) &&
                   reinterpret_cast<uintptr_t>(M) % align == 0 &&
                   (SRC != 0 || reinterpret_cast<uintptr_t>(G) % 32 == 0);
  dim3 grid(static_cast<unsigned>(C_pad / kTC), static_cast<unsigned>(R_pad / kTR), static_cast<unsigned>(g.batch));
#ifdef MC_DEBUG
  // every grid below writes one partial per block: the workspace holds
  // prescale_tiles per matrix
  if ((C_pad / kTC) * (R_pad / kTR) != g.prescale_tiles || (C_pad / kSC) * (R_pad / kSR) != g.prescale_tiles)
    return hipErrorInvalidValue;
#endif
  if (vec && S != nullptr)
    hipLaunchKernelGGL(momentum_prescale_rows_kernel<SRC>,
                       dim3(static_cast<unsigned>(C_pad / kSC), static_cast<unsigned>(R_pad / kSR),
                            static_cast<unsigned>(g.batch)),
                       dim3(kThreads), 0, stream, M, G, batch_stride, mu, R, C, R_pad, C_pad, S, SL, partials);
  else if (vec)
    hipLaunchKernelGGL((momentum_prescale_kernel<true, SRC>), grid, dim3(kThreads), 0, stream, M, G, batch_stride,
                       mu, R, C, R_pad, C_pad, S, T, SL, TL, partials);
  else
    hipLaunchKernelGGL((momentum_prescale_kernel<false, SRC>), grid, dim3(kThreads), 0, stream, M, G,
                       batch_stride, mu, R, C, R_pad, C_pad, S, T, SL, TL, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(invnorm_kernel, dim3(static_cast<unsigned>(g.batch)), dim3(kThreads), 0, stream, partials,
                     g.prescale_tiles, eps, invnorm);
  return hipGetLastError();
}
}  // namespace

MC_DEBUG_UNIT(ns_prep)

hipError_t launch_momentum_prescale(float* M, const float* G, int64_t batch_stride, float mu,
                                    const NsGeometry& g, float eps, char* ws, hipStream_t stream) {
  return launch_prescale_unscaled<0>(M, G, batch_stride, mu, g, eps, ws, stream);
}

hipError_t launch_ns_prescale_unscaled(const void* M, bool m_bf16, int64_t m_batch_stride, const NsGeometry& g,
                                       float eps, char* ws, hipStream_t stream) {
  void* Mv = const_cast<void*>(M);  // read only for SRC 1 and 2
  if (m_bf16) return launch_prescale_unscaled<2>(Mv, nullptr, m_batch_stride, 0.f, g, eps, ws, stream);
  return launch_prescale_unscaled<1>(Mv, nullptr, m_batch_stride, 0.f, g, eps, ws, stream);
}


}  // namespace mc
