// Newton-Schulz input and output stages.
//
//   norm      ||M_b||_F per matrix: float32 partial sums of squares per chunk,
//             then one block per matrix combines them in double in a fixed
//             order (deterministic), giving inv_b = 1 / (||M_b||_F + eps).
//   prescale  X_0 = bf16(inv_b * M_b), or of M_b^T when rows > cols, written
//             into the zero-padded n_pad x m_pad workspace layout the GEMMs
//             use.
//   output    O_b = out_scale * X (or X^T), cast to the output dtype.
//   momentum + pre-scale (the fused step): M_b <- mu M_b + G_b in place, and
//             in the same pass X_0 = bf16(M_b) unscaled plus per-tile partial
//             sums of squares of the new M_b; the 1 / (||M_b||_F + eps) is
//             applied inside the first Newton-Schulz step's GEMM epilogues.
// Both move 8-element runs (16-byte vectors where the row length and the
// alignment allow); the transposing variants go through a 64 x 64 LDS tile so
// both the read and the write side are coalesced.

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {

namespace {
constexpr int kThreads = 256;
constexpr int64_t kNormChunk = 32768;  // elements per partial sum
constexpr int kT = 64;                 // transpose tile
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
  g.sumsq_chunks = (rows * cols + kNormChunk - 1) / kNormChunk;
  g.prescale_tiles = (g.n_pad / kT) * (g.m_pad / kT);
  const size_t xb = static_cast<size_t>(batch) * g.n_pad * g.m_pad * 2;
  const size_t ab = static_cast<size_t>(batch) * g.n_pad * g.n_pad * 2;
  size_t off = 0;
  g.off_x0 = off; off = align256(off + xb);
  g.off_x1 = off; off = align256(off + xb);
  g.off_a = off; off = align256(off + ab);
  g.off_b = off; off = align256(off + ab);
  const int64_t partials = g.sumsq_chunks > g.prescale_tiles ? g.sumsq_chunks : g.prescale_tiles;
  g.off_partials = off; off = align256(off + static_cast<size_t>(batch * partials) * 4);
  g.off_invnorm = off; off = align256(off + static_cast<size_t>(batch) * 4);
  g.total = off;
  return g;
}

namespace {

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

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

// grid (chunks, batch)
template <bool BF16>
__global__ __launch_bounds__(kThreads) void sumsq_kernel(const void* __restrict__ M,
                                                        int64_t batch_stride, int64_t count,
                                                        int64_t chunks, float* __restrict__ partials) {
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.y;
  const char* base = static_cast<const char*>(M) + static_cast<size_t>(b * batch_stride) * (BF16 ? 2 : 4);
  const int64_t begin = blockIdx.x * kNormChunk;
  const int64_t end = min(count, begin + kNormChunk);
  float acc = 0.f;
  for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) {
    const float x = load_elem<BF16>(base, i);
    acc = fmaf(x, x, acc);
  }
  const float s = block_sum(acc, red);
  if (threadIdx.x == 0) partials[b * chunks + blockIdx.x] = s;
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

// Pre-scale.  M_b is R x C (rows x cols); it is scaled by
// inv_b = 1 / (||M_b||_F + eps), rounded once to bf16 and written zero-padded
// either as it is into S (R_pad x C_pad; rows <= cols: X_0 = M) or transposed
// into T (C_pad x R_pad; rows > cols: X_0 = M^T); the other pointer is null.
// grid (C_pad / 64, R_pad / 64, batch); each block reads one 64 x 64 tile in
// 8-element runs (vector loads when VEC) and writes it straight from
// registers or transposed through LDS.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void prescale_kernel(const void* __restrict__ M, int64_t batch_stride,
                                                           int64_t R, int64_t C, int64_t R_pad,
                                                           int64_t C_pad, const float* __restrict__ invnorm,
                                                           uint16_t* __restrict__ S,
                                                           uint16_t* __restrict__ T) {
  __shared__ float tile[kT][kT + 1];
  const int64_t b = blockIdx.z;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kT, r0 = static_cast<int64_t>(blockIdx.y) * kT;
  const float inv = invnorm[b];
  const char* base = static_cast<const char*>(M) + static_cast<size_t>(b * batch_stride) * (BF16 ? 2 : 4);
  uint16_t* sb = S + static_cast<size_t>(b) * R_pad * C_pad;
  uint16_t* tb = T + static_cast<size_t>(b) * R_pad * C_pad;
  const int q = threadIdx.x & 7;  // 8-element run within a row
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rr = pass * 32 + (threadIdx.x >> 3);
    const int64_t r = r0 + rr, c = c0 + 8 * q;
    float x[8];
    if constexpr (VEC) {
      // C % 8 == 0: a run is wholly inside or wholly outside the matrix
      if (r < R && c < C) {
        if constexpr (BF16) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(base + (r * C + c) * 2);
          x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
          x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
        } else {
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(base + (r * C + c) * 4);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(base + (r * C + c + 4) * 4);
          x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
          x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= inv;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (r < R && c + e < C) ? load_elem<BF16>(base, r * C + c + e) * inv : 0.f;
    }
    if (S != nullptr) {
      const u32x4 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7])};
      *reinterpret_cast<u32x4*>(sb + x_off(r, c, R_pad)) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rr][8 * q + e] = x[e];
    }
  }
  if (S != nullptr) return;
  __syncthreads();
  // T[c0 + cc][r0 + 8 q' .. + 7] = tile[8 q' ..][cc]
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cc = pass * 32 + (threadIdx.x >> 3);
    const int rq = 8 * q;
    const u32x4 o = {pack_bf16x2(tile[rq + 0][cc], tile[rq + 1][cc]), pack_bf16x2(tile[rq + 2][cc], tile[rq + 3][cc]),
                     pack_bf16x2(tile[rq + 4][cc], tile[rq + 5][cc]), pack_bf16x2(tile[rq + 6][cc], tile[rq + 7][cc])};
    *reinterpret_cast<u32x4*>(tb + x_off(c0 + cc, r0 + rq, C_pad)) = o;
  }
}

// Fused momentum and pre-scale.  M_b, G_b are R x C float32 (rows x cols);
// M_b <- fl32(fl32(mu M_b) + G_b) in place (bit-identical to the stand-alone
// momentum), and the new M_b is written unscaled as bf16 into S (R_pad x
// C_pad) or transposed into T (C_pad x R_pad), zero-padded, as in
// prescale_kernel.  Each block also writes the float32 sum of squares of its
// tile's new M values to partials[b * tiles + tile].
// grid (C_pad / 64, R_pad / 64, batch).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void momentum_prescale_kernel(float* __restrict__ M,
                                                                    const float* __restrict__ G,
                                                                    int64_t batch_stride, float mu, int64_t R,
                                                                    int64_t C, int64_t R_pad, int64_t C_pad,
                                                                    uint16_t* __restrict__ S,
                                                                    uint16_t* __restrict__ T,
                                                                    float* __restrict__ partials) {
  __shared__ float tile[kT][kT + 1];
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.z;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kT, r0 = static_cast<int64_t>(blockIdx.y) * kT;
  float* mb = M + b * batch_stride;
  const float* gb = G + b * batch_stride;
  uint16_t* sb = S + static_cast<size_t>(b) * R_pad * C_pad;
  uint16_t* tb = T + static_cast<size_t>(b) * R_pad * C_pad;
  const int q = threadIdx.x & 7;
  float ss = 0.f;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rr = pass * 32 + (threadIdx.x >> 3);
    const int64_t r = r0 + rr, c = c0 + 8 * q;
    float x[8];
    if constexpr (VEC) {
      // C % 8 == 0: a run is wholly inside or wholly outside the matrix
      if (r < R && c < C) {
        f32x4* mp = reinterpret_cast<f32x4*>(mb + r * C + c);
        const f32x4* gp = reinterpret_cast<const f32x4*>(gb + r * C + c);
        f32x4 m0 = __builtin_nontemporal_load(mp), m1 = __builtin_nontemporal_load(mp + 1);
        const f32x4 g0 = __builtin_nontemporal_load(gp), g1 = __builtin_nontemporal_load(gp + 1);
        m0.x = momentum_op(m0.x, g0.x, mu);
        m0.y = momentum_op(m0.y, g0.y, mu);
        m0.z = momentum_op(m0.z, g0.z, mu);
        m0.w = momentum_op(m0.w, g0.w, mu);
        m1.x = momentum_op(m1.x, g1.x, mu);
        m1.y = momentum_op(m1.y, g1.y, mu);
        m1.z = momentum_op(m1.z, g1.z, mu);
        m1.w = momentum_op(m1.w, g1.w, mu);
        __builtin_nontemporal_store(m0, mp);
        __builtin_nontemporal_store(m1, mp + 1);
        x[0] = m0.x; x[1] = m0.y; x[2] = m0.z; x[3] = m0.w;
        x[4] = m1.x; x[5] = m1.y; x[6] = m1.z; x[7] = m1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = 0.f;
        if (r < R && c + e < C) {
          const float m = momentum_op(mb[r * C + c + e], gb[r * C + c + e], mu);
          mb[r * C + c + e] = m;
          x[e] = m;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    if (S != nullptr) {
      const u32x4 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7])};
      *reinterpret_cast<u32x4*>(sb + x_off(r, c, R_pad)) = o;
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
  for (int pass = 0; pass < 2; ++pass) {
    const int cc = pass * 32 + (threadIdx.x >> 3);
    const int rq = 8 * q;
    const u32x4 o = {pack_bf16x2(tile[rq + 0][cc], tile[rq + 1][cc]), pack_bf16x2(tile[rq + 2][cc], tile[rq + 3][cc]),
                     pack_bf16x2(tile[rq + 4][cc], tile[rq + 5][cc]), pack_bf16x2(tile[rq + 6][cc], tile[rq + 7][cc])};
    *reinterpret_cast<u32x4*>(tb + x_off(c0 + cc, r0 + rq, C_pad)) = o;
  }
}

// The same for rows <= cols with 16-byte aligned rows (the common case),
// with row strips instead of square tiles: a block covers 16 rows x 256
// columns (one column panel of X), so every row segment it reads is 1 KB of
// M and of G and every X_0 segment it writes is 512 contiguous bytes.
// grid (C_pad / 256, R_pad / 16, batch); 4096 elements per block, like the
// 64 x 64 tiles, so the partial-sum count per matrix is the same.
__global__ __launch_bounds__(kThreads) void momentum_prescale_rows_kernel(
    float* __restrict__ M, const float* __restrict__ G, int64_t batch_stride, float mu, int64_t R, int64_t C,
    int64_t R_pad, int64_t C_pad, uint16_t* __restrict__ X0, float* __restrict__ partials) {
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.z;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + 8 * (threadIdx.x & 31);
  float* mb = M + b * batch_stride;
  const float* gb = G + b * batch_stride;
  uint16_t* xb = X0 + static_cast<size_t>(b) * R_pad * C_pad;
  float ss = 0.f;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t r = static_cast<int64_t>(blockIdx.y) * 16 + pass * 8 + (threadIdx.x >> 5);
    float x[8];
    if (r < R && c < C) {  // C % 8 == 0: a run is wholly inside or outside
      f32x4* mp = reinterpret_cast<f32x4*>(mb + r * C + c);
      const f32x4* gp = reinterpret_cast<const f32x4*>(gb + r * C + c);
      f32x4 m0 = __builtin_nontemporal_load(mp), m1 = __builtin_nontemporal_load(mp + 1);
      const f32x4 g0 = __builtin_nontemporal_load(gp), g1 = __builtin_nontemporal_load(gp + 1);
      m0.x = momentum_op(m0.x, g0.x, mu);
      m0.y = momentum_op(m0.y, g0.y, mu);
      m0.z = momentum_op(m0.z, g0.z, mu);
      m0.w = momentum_op(m0.w, g0.w, mu);
      m1.x = momentum_op(m1.x, g1.x, mu);
      m1.y = momentum_op(m1.y, g1.y, mu);
      m1.z = momentum_op(m1.z, g1.z, mu);
      m1.w = momentum_op(m1.w, g1.w, mu);
      __builtin_nontemporal_store(m0, mp);
      __builtin_nontemporal_store(m1, mp + 1);
      x[0] = m0.x; x[1] = m0.y; x[2] = m0.z; x[3] = m0.w;
      x[4] = m1.x; x[5] = m1.y; x[6] = m1.z; x[7] = m1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    const u32x4 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    *reinterpret_cast<u32x4*>(xb + x_off(r, c, R_pad)) = o;
  }
  const float block_ss = block_sum(ss, red);
  if (threadIdx.x == 0) partials[b * gridDim.x * gridDim.y + blockIdx.y * gridDim.x + blockIdx.x] = block_ss;
}

template <bool OBF16>
__device__ __forceinline__ void store_out(void* O, int64_t idx, float v) {
  if constexpr (OBF16) static_cast<uint16_t*>(O)[idx] = f32_to_bf16(v);
  else static_cast<float*>(O)[idx] = v;
}

// Output, element by element: O[r][c] = s * X[r][c] (X in the panel layout).
// grid (ceil(R * C / 256), batch)
template <bool OBF16>
__global__ __launch_bounds__(kThreads) void output_kernel(const uint16_t* __restrict__ src, int64_t R,
                                                         int64_t C, int64_t n_pad, int64_t src_stride,
                                                         void* __restrict__ O, int64_t o_stride, float s) {
  const int64_t b = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= R * C) return;
  const int64_t r = e / C, c = e % C;
  const float x = bf16_to_f32(src[b * src_stride + x_off(r, c, n_pad)]);
  char* ob = static_cast<char*>(O) + static_cast<size_t>(b * o_stride) * (OBF16 ? 2 : 4);
  store_out<OBF16>(ob, e, x * s);
}

// Output, 8 elements per thread (C % 8 == 0 and 16-byte aligned rows of O).
// grid (ceil(R * C / 8 / 256), batch)
template <bool OBF16>
__global__ __launch_bounds__(kThreads) void output_vec_kernel(const uint16_t* __restrict__ src, int64_t R,
                                                             int64_t C, int64_t n_pad, int64_t src_stride,
                                                             void* __restrict__ O, int64_t o_stride,
                                                             float s) {
  const int64_t b = blockIdx.y;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_row = C / 8;
  if (v >= R * per_row) return;
  const int64_t r = v / per_row, c = (v % per_row) * 8;
  const u32x4 x = *reinterpret_cast<const u32x4*>(src + b * src_stride + x_off(r, c, n_pad));
  const float y[8] = {bf16_lo(x.x) * s, bf16_hi(x.x) * s, bf16_lo(x.y) * s, bf16_hi(x.y) * s,
                      bf16_lo(x.z) * s, bf16_hi(x.z) * s, bf16_lo(x.w) * s, bf16_hi(x.w) * s};
  char* ob = static_cast<char*>(O) + static_cast<size_t>(b * o_stride + r * C + c) * (OBF16 ? 2 : 4);
  if constexpr (OBF16) {
    const u32x4 o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                     pack_bf16x2(y[6], y[7])};
    *reinterpret_cast<u32x4*>(ob) = o;
  } else {
    const f32x4 o0 = {y[0], y[1], y[2], y[3]}, o1 = {y[4], y[5], y[6], y[7]};
    reinterpret_cast<f32x4*>(ob)[0] = o0;
    reinterpret_cast<f32x4*>(ob)[1] = o1;
  }
}

// Transposing output (rows > cols): O[r][c] = s * X[c][r], O is R x C =
// m x n, X is n_pad x m_pad in the panel layout.  grid (R_pad / 64, C_pad / 64, batch): each block
// reads 64 rows x 64 columns of X in 16-byte runs and writes the transposed
// 64 x 64 block of O, in 8-element runs when VEC (C % 8 == 0 and 16-byte
// aligned rows), else element by element.
template <bool OBF16, bool VEC>
__global__ __launch_bounds__(kThreads) void output_t_kernel(const uint16_t* __restrict__ X, int64_t R,
                                                           int64_t C, int64_t n_pad, int64_t src_stride,
                                                           void* __restrict__ O, int64_t o_stride,
                                                           float s) {
  __shared__ float tile[kT][kT + 1];
  const int64_t b = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kT, c0 = static_cast<int64_t>(blockIdx.y) * kT;
  const uint16_t* xb = X + b * src_stride;
  const int q = threadIdx.x & 7;
  // tile[cc][rr] = X[c0 + cc][r0 + rr]
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cc = pass * 32 + (threadIdx.x >> 3);
    const u32x4 v = *reinterpret_cast<const u32x4*>(xb + x_off(c0 + cc, r0 + 8 * q, n_pad));
    tile[cc][8 * q + 0] = bf16_lo(v.x) * s;
    tile[cc][8 * q + 1] = bf16_hi(v.x) * s;
    tile[cc][8 * q + 2] = bf16_lo(v.y) * s;
    tile[cc][8 * q + 3] = bf16_hi(v.y) * s;
    tile[cc][8 * q + 4] = bf16_lo(v.z) * s;
    tile[cc][8 * q + 5] = bf16_hi(v.z) * s;
    tile[cc][8 * q + 6] = bf16_lo(v.w) * s;
    tile[cc][8 * q + 7] = bf16_hi(v.w) * s;
  }
  __syncthreads();
  char* ob = static_cast<char*>(O) + static_cast<size_t>(b * o_stride) * (OBF16 ? 2 : 4);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rr = pass * 32 + (threadIdx.x >> 3);
    const int64_t r = r0 + rr, c = c0 + 8 * q;
    if (r >= R) continue;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = tile[8 * q + e][rr];
    if constexpr (VEC) {
      if (c >= C) continue;  // C % 8 == 0: the run is wholly in or out
      char* dst = ob + (r * C + c) * (OBF16 ? 2 : 4);
      if constexpr (OBF16) {
        const u32x4 o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                         pack_bf16x2(y[6], y[7])};
        *reinterpret_cast<u32x4*>(dst) = o;
      } else {
        const f32x4 o0 = {y[0], y[1], y[2], y[3]}, o1 = {y[4], y[5], y[6], y[7]};
        reinterpret_cast<f32x4*>(dst)[0] = o0;
        reinterpret_cast<f32x4*>(dst)[1] = o1;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < C) store_out<OBF16>(ob, r * C + c + e, y[e]);
    }
  }
}

}  // namespace

hipError_t launch_ns_norm(const void* M, bool m_bf16, int64_t m_batch_stride, const NsGeometry& g,
                          float eps, char* ws, hipStream_t stream) {
  float* partials = reinterpret_cast<float*>(ws + g.off_partials);
  float* invnorm = reinterpret_cast<float*>(ws + g.off_invnorm);
  dim3 grid(static_cast<unsigned>(g.sumsq_chunks), static_cast<unsigned>(g.batch));
  if (m_bf16)
    hipLaunchKernelGGL(sumsq_kernel<true>, grid, dim3(kThreads), 0, stream, M, m_batch_stride,
                       g.rows * g.cols, g.sumsq_chunks, partials);
  else
    hipLaunchKernelGGL(sumsq_kernel<false>, grid, dim3(kThreads), 0, stream, M, m_batch_stride,
                       g.rows * g.cols, g.sumsq_chunks, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(invnorm_kernel, dim3(static_cast<unsigned>(g.batch)), dim3(kThreads), 0, stream,
                     partials, g.sumsq_chunks, eps, invnorm);
  return hipGetLastError();
}

hipError_t launch_ns_prescale(const void* M, bool m_bf16, int64_t m_batch_stride,
                              const NsGeometry& g, char* ws, hipStream_t stream) {
  const float* invnorm = reinterpret_cast<const float*>(ws + g.off_invnorm);
  uint16_t* X0 = reinterpret_cast<uint16_t*>(ws + g.off_x0);
  // M is R x C = rows x cols; X_0 = M (straight) or M^T (transposed)
  const int64_t R = g.rows, C = g.cols;
  const int64_t R_pad = g.transposed ? g.m_pad : g.n_pad, C_pad = g.transposed ? g.n_pad : g.m_pad;
  uint16_t* S = g.transposed ? nullptr : X0;
  uint16_t* T = g.transposed ? X0 : nullptr;
  const size_t esz = m_bf16 ? 2 : 4;
  const bool vec = C % 8 == 0 && (g.batch == 1 || m_batch_stride % 8 == 0) &&
                   reinterpret_cast<uintptr_t>(M) % (8 * esz) == 0;
  dim3 grid(static_cast<unsigned>(C_pad / kT), static_cast<unsigned>(R_pad / kT), static_cast<unsigned>(g.batch));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, M, m_batch_stride, R, C, R_pad, C_pad, invnorm,
                       S, T);
  };
  if (m_bf16) {
    if (vec) go(prescale_kernel<true, true>);
    else go(prescale_kernel<true, false>);
  } else {
    if (vec) go(prescale_kernel<false, true>);
    else go(prescale_kernel<false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_momentum_prescale(float* M, const float* G, int64_t batch_stride, float mu,
                                    const NsGeometry& g, float eps, char* ws, hipStream_t stream) {
  float* partials = reinterpret_cast<float*>(ws + g.off_partials);
  float* invnorm = reinterpret_cast<float*>(ws + g.off_invnorm);
  uint16_t* X0 = reinterpret_cast<uint16_t*>(ws + g.off_x0);
  const int64_t R = g.rows, C = g.cols;
  const int64_t R_pad = g.transposed ? g.m_pad : g.n_pad, C_pad = g.transposed ? g.n_pad : g.m_pad;
  uint16_t* S = g.transposed ? nullptr : X0;
  uint16_t* T = g.transposed ? X0 : nullptr;
  const bool vec = C % 8 == 0 && (g.batch == 1 || batch_stride % 8 == 0) &&
                   reinterpret_cast<uintptr_t>(M) % 32 == 0 && reinterpret_cast<uintptr_t>(G) % 32 == 0;
  dim3 grid(static_cast<unsigned>(C_pad / kT), static_cast<unsigned>(R_pad / kT), static_cast<unsigned>(g.batch));
  if (vec && S != nullptr)
    hipLaunchKernelGGL(momentum_prescale_rows_kernel,
                       dim3(static_cast<unsigned>(C_pad / 256), static_cast<unsigned>(R_pad / 16),
                            static_cast<unsigned>(g.batch)),
                       dim3(kThreads), 0, stream, M, G, batch_stride, mu, R, C, R_pad, C_pad, S, partials);
  else if (vec)
    hipLaunchKernelGGL(momentum_prescale_kernel<true>, grid, dim3(kThreads), 0, stream, M, G, batch_stride, mu, R, C,
                       R_pad, C_pad, S, T, partials);
  else
    hipLaunchKernelGGL(momentum_prescale_kernel<false>, grid, dim3(kThreads), 0, stream, M, G, batch_stride, mu, R,
                       C, R_pad, C_pad, S, T, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(invnorm_kernel, dim3(static_cast<unsigned>(g.batch)), dim3(kThreads), 0, stream, partials,
                     g.prescale_tiles, eps, invnorm);
  return hipGetLastError();
}

hipError_t launch_ns_output(const uint16_t* X, const NsGeometry& g, void* O, bool o_bf16,
                            int64_t o_batch_stride, float out_scale, hipStream_t stream) {
  const int64_t R = g.rows, C = g.cols;
  const int64_t src_stride = g.n_pad * g.m_pad;
  const bool vec = C % 8 == 0 && (g.batch == 1 || o_batch_stride % 8 == 0) &&
                   reinterpret_cast<uintptr_t>(O) % 16 == 0;
  if (g.transposed) {
    dim3 grid(static_cast<unsigned>(g.m_pad / kT), static_cast<unsigned>(g.n_pad / kT),
              static_cast<unsigned>(g.batch));
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, X, R, C, g.n_pad, src_stride, O, o_batch_stride,
                         out_scale);
    };
    if (o_bf16) {
      if (vec) go(output_t_kernel<true, true>);
      else go(output_t_kernel<true, false>);
    } else {
      if (vec) go(output_t_kernel<false, true>);
      else go(output_t_kernel<false, false>);
    }
  } else if (vec) {
    const int64_t vecs = R * C / 8;
    dim3 grid(static_cast<unsigned>((vecs + kThreads - 1) / kThreads), static_cast<unsigned>(g.batch));
    if (o_bf16)
      hipLaunchKernelGGL(output_vec_kernel<true>, grid, dim3(kThreads), 0, stream, X, R, C, g.n_pad, src_stride, O,
                         o_batch_stride, out_scale);
    else
      hipLaunchKernelGGL(output_vec_kernel<false>, grid, dim3(kThreads), 0, stream, X, R, C, g.n_pad, src_stride,
                         O, o_batch_stride, out_scale);
  } else {
    const int64_t count = R * C;
    dim3 grid(static_cast<unsigned>((count + kThreads - 1) / kThreads), static_cast<unsigned>(g.batch));
    if (o_bf16)
      hipLaunchKernelGGL(output_kernel<true>, grid, dim3(kThreads), 0, stream, X, R, C, g.n_pad, src_stride, O,
                         o_batch_stride, out_scale);
    else
      hipLaunchKernelGGL(output_kernel<false>, grid, dim3(kThreads), 0, stream, X, R, C, g.n_pad, src_stride, O,
                         o_batch_stride, out_scale);
  }
  return hipGetLastError();
}

}  // namespace mc
