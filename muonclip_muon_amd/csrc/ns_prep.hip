// Newton-Schulz input and output stages.
//
//   norm      ||M_b||_F per matrix: float32 partial sums of squares per chunk,
//             then one block per matrix combines them in double in a fixed
//             order (deterministic), giving inv_b = 1 / (||M_b||_F + eps).
//   prescale  X_0 = bf16(inv_b * M_b), or of M_b^T when rows > cols, written
//             into the zero-padded n_pad x m_pad workspace layout the GEMMs use.
//   output    O_b = out_scale * X (or X^T), cast to the output dtype.
// The transposing variants go through a 64 x 64 LDS tile so both the read
// and the write side are coalesced.

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
  const size_t xb = static_cast<size_t>(batch) * g.n_pad * g.m_pad * 2;
  const size_t ab = static_cast<size_t>(batch) * g.n_pad * g.n_pad * 2;
  size_t off = 0;
  g.off_x0 = off; off = align256(off + xb);
  g.off_x1 = off; off = align256(off + xb);
  g.off_a = off; off = align256(off + ab);
  g.off_b = off; off = align256(off + ab);
  g.off_partials = off; off = align256(off + static_cast<size_t>(batch * g.sumsq_chunks) * 4);
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

// Straight pre-scale (rows <= cols): X0[i][k] = bf16(inv * M[i][k]); one
// thread per 8 consecutive k of the padded row.  grid (ceil(n_pad*m_pad/8/256), batch)
template <bool BF16>
__global__ __launch_bounds__(kThreads) void prescale_kernel(const void* __restrict__ M,
                                                           int64_t batch_stride, int64_t n, int64_t m,
                                                           int64_t n_pad, int64_t m_pad,
                                                           const float* __restrict__ invnorm,
                                                           uint16_t* __restrict__ X0) {
  const int64_t b = blockIdx.y;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_row = m_pad / 8;
  if (v >= n_pad * per_row) return;
  const int64_t i = v / per_row, k = (v % per_row) * 8;
  const float inv = invnorm[b];
  const char* base = static_cast<const char*>(M) + static_cast<size_t>(b * batch_stride) * (BF16 ? 2 : 4);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x[e] = (i < n && k + e < m) ? load_elem<BF16>(base, i * m + k + e) * inv : 0.f;
  u32x4 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  *reinterpret_cast<u32x4*>(X0 + static_cast<size_t>(b) * n_pad * m_pad + i * m_pad + k) = o;
}

// Transposing pre-scale (rows > cols): X0[i][k] = bf16(inv * M[k][i]) with M
// rows x cols = m x n.  grid (m_pad/64, n_pad/64, batch); tile over (k, i).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void prescale_t_kernel(const void* __restrict__ M,
                                                             int64_t batch_stride, int64_t n,
                                                             int64_t m, int64_t n_pad, int64_t m_pad,
                                                             const float* __restrict__ invnorm,
                                                             uint16_t* __restrict__ X0) {
  __shared__ float tile[kT][kT + 1];
  const int64_t b = blockIdx.z;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kT, i0 = static_cast<int64_t>(blockIdx.y) * kT;
  const float inv = invnorm[b];
  const char* base = static_cast<const char*>(M) + static_cast<size_t>(b * batch_stride) * (BF16 ? 2 : 4);
  // read M[k0 + r][i0 + c] (row r of the tile is a row of M; M has n columns)
  for (int t = threadIdx.x; t < kT * kT; t += kThreads) {
    const int r = t / kT, c = t % kT;
    const int64_t k = k0 + r, i = i0 + c;
    tile[r][c] = (k < m && i < n) ? load_elem<BF16>(base, k * n + i) * inv : 0.f;
  }
  __syncthreads();
  // write X0[i0 + r][k0 + c .. +7] = tile[c..][r]
  uint16_t* xb = X0 + static_cast<size_t>(b) * n_pad * m_pad;
  for (int t = threadIdx.x; t < kT * kT / 8; t += kThreads) {
    const int r = t / (kT / 8), c = (t % (kT / 8)) * 8;
    u32x4 o = {pack_bf16x2(tile[c + 0][r], tile[c + 1][r]), pack_bf16x2(tile[c + 2][r], tile[c + 3][r]),
               pack_bf16x2(tile[c + 4][r], tile[c + 5][r]), pack_bf16x2(tile[c + 6][r], tile[c + 7][r])};
    *reinterpret_cast<u32x4*>(xb + (i0 + r) * m_pad + k0 + c) = o;
  }
}

template <bool OBF16>
__device__ __forceinline__ void store_out(void* O, int64_t idx, float v) {
  if constexpr (OBF16) static_cast<uint16_t*>(O)[idx] = f32_to_bf16(v);
  else static_cast<float*>(O)[idx] = v;
}

// Straight output: O[r][c] = s * X[r][c], r < rows = n, c < cols = m.
// grid (ceil(rows*cols/256), batch)
template <bool OBF16>
__global__ __launch_bounds__(kThreads) void output_kernel(const uint16_t* __restrict__ X, int64_t n,
                                                         int64_t m, int64_t n_pad, int64_t m_pad,
                                                         void* __restrict__ O, int64_t o_stride,
                                                         float s) {
  const int64_t b = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= n * m) return;
  const int64_t r = e / m, c = e % m;
  const float x = bf16_to_f32(X[static_cast<size_t>(b) * n_pad * m_pad + r * m_pad + c]);
  char* ob = static_cast<char*>(O) + static_cast<size_t>(b * o_stride) * (OBF16 ? 2 : 4);
  store_out<OBF16>(ob, e, x * s);
}

// Transposing output: O[r][c] = s * X[c][r], O is rows x cols = m x n.
// grid (m_pad/64, n_pad/64, batch); tile over (c in X rows, r in X cols).
template <bool OBF16>
__global__ __launch_bounds__(kThreads) void output_t_kernel(const uint16_t* __restrict__ X, int64_t n,
                                                           int64_t m, int64_t n_pad, int64_t m_pad,
                                                           void* __restrict__ O, int64_t o_stride,
                                                           float s) {
  __shared__ float tile[kT][kT + 1];
  const int64_t b = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kT, c0 = static_cast<int64_t>(blockIdx.y) * kT;
  const uint16_t* xb = X + static_cast<size_t>(b) * n_pad * m_pad;
  // tile[cc][rr] = X[c0 + cc][r0 + rr]
  for (int t = threadIdx.x; t < kT * kT; t += kThreads) {
    const int cc = t / kT, rr = t % kT;
    tile[cc][rr] = bf16_to_f32(xb[(c0 + cc) * m_pad + r0 + rr]);
  }
  __syncthreads();
  char* ob = static_cast<char*>(O) + static_cast<size_t>(b * o_stride) * (OBF16 ? 2 : 4);
  for (int t = threadIdx.x; t < kT * kT; t += kThreads) {
    const int rr = t / kT, cc = t % kT;
    const int64_t r = r0 + rr, c = c0 + cc;
    if (r < m && c < n) store_out<OBF16>(ob, r * n + c, tile[cc][rr] * s);
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
  if (!g.transposed) {
    const int64_t vecs = g.n_pad * g.m_pad / 8;
    dim3 grid(static_cast<unsigned>((vecs + kThreads - 1) / kThreads), static_cast<unsigned>(g.batch));
    if (m_bf16)
      hipLaunchKernelGGL(prescale_kernel<true>, grid, dim3(kThreads), 0, stream, M, m_batch_stride, g.n,
                         g.m, g.n_pad, g.m_pad, invnorm, X0);
    else
      hipLaunchKernelGGL(prescale_kernel<false>, grid, dim3(kThreads), 0, stream, M, m_batch_stride,
                         g.n, g.m, g.n_pad, g.m_pad, invnorm, X0);
  } else {
    dim3 grid(static_cast<unsigned>(g.m_pad / kT), static_cast<unsigned>(g.n_pad / kT),
              static_cast<unsigned>(g.batch));
    if (m_bf16)
      hipLaunchKernelGGL(prescale_t_kernel<true>, grid, dim3(kThreads), 0, stream, M, m_batch_stride,
                         g.n, g.m, g.n_pad, g.m_pad, invnorm, X0);
    else
      hipLaunchKernelGGL(prescale_t_kernel<false>, grid, dim3(kThreads), 0, stream, M, m_batch_stride,
                         g.n, g.m, g.n_pad, g.m_pad, invnorm, X0);
  }
  return hipGetLastError();
}

hipError_t launch_ns_output(const uint16_t* X, const NsGeometry& g, void* O, bool o_bf16,
                            int64_t o_batch_stride, float out_scale, hipStream_t stream) {
  if (!g.transposed) {
    const int64_t count = g.n * g.m;
    dim3 grid(static_cast<unsigned>((count + kThreads - 1) / kThreads), static_cast<unsigned>(g.batch));
    if (o_bf16)
      hipLaunchKernelGGL(output_kernel<true>, grid, dim3(kThreads), 0, stream, X, g.n, g.m, g.n_pad,
                         g.m_pad, O, o_batch_stride, out_scale);
    else
      hipLaunchKernelGGL(output_kernel<false>, grid, dim3(kThreads), 0, stream, X, g.n, g.m, g.n_pad,
                         g.m_pad, O, o_batch_stride, out_scale);
  } else {
    dim3 grid(static_cast<unsigned>(g.m_pad / kT), static_cast<unsigned>(g.n_pad / kT),
              static_cast<unsigned>(g.batch));
    if (o_bf16)
      hipLaunchKernelGGL(output_t_kernel<true>, grid, dim3(kThreads), 0, stream, X, g.n, g.m, g.n_pad,
                         g.m_pad, O, o_batch_stride, out_scale);
    else
      hipLaunchKernelGGL(output_t_kernel<false>, grid, dim3(kThreads), 0, stream, X, g.n, g.m,
                         g.n_pad, g.m_pad, O, o_batch_stride, out_scale);
  }
  return hipGetLastError();
}

}  // namespace mc
