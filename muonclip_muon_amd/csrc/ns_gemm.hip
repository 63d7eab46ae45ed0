// Batched bf16 MFMA GEMMs of one Newton-Schulz step (gfx950).
//
// One step of the odd polynomial p(X) = a X + b (X X^T) X + c (X X^T)^2 X is
// three GEMMs on the zero-padded n_pad x m_pad bf16 state X:
//   mode 0  A  = X X^T              K = m_pad   (out n_pad x n_pad)
//   mode 1  B  = b A + c A A        K = n_pad   (A is symmetric, so A A = A A^T)
//   mode 2  X' = a X + B X          K = n_pad   (out n_pad x m_pad)
// All three accumulate in float32 on v_mfma_f32_32x32x16_bf16 and round the
// epilogue result once to bf16.
//
// Tiling: a 256-thread workgroup (4 wave64s, 2 x 2) owns a 256 x 256 output
// tile; each wave owns 128 x 128 = 4 x 4 MFMA tiles of 32 x 32 (256 float32
// accumulators per lane).  The K loop steps by 64 through a double-buffered
// LDS stage of two 256 x 64 bf16 operand tiles (64 KB per stage); the next
// stage's global loads are issued before the current stage's MFMAs.
//
// Operand layout in LDS: every operand tile is stored "K-contiguous": row r
// (an output row or column index) holds 64 consecutive k as 8 units of
// 16 bytes, unit u stored at position u ^ (r & 7) (XOR swizzle: the 8 lanes
// that share a ds_read_b128 phase touch 8 different 16-byte bank groups).
// Modes 0/1 read both operands K-contiguous from global memory.  In mode 2
// the right operand X is row-major with K as its row index, so each thread
// loads an 8 (k) x 8 (column) bf16 block, transposes it in registers with
// v_perm_b32 and writes 8 K-contiguous rows.
//
// MFMA operand roles: the MFMA "A" operand is the right-hand tile (output
// columns j) and "B" is the left-hand tile (output rows i), so that each lane
// ends up holding 4 consecutive j of one output row i per 4-register group:
// the epilogue then reads and writes 8-byte runs.
// Lane layout of v_mfma_f32_32x32x16_bf16 (measured on gfx950): A/B lane l
// holds row/column l % 32, k = 8 * (l / 32) + [0, 8); result register r of
// lane l is row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 256;
constexpr int kUnits = kBK / 8;  // 16-byte units per LDS row

struct Lds {
  u32x4 p[2][kBM][kUnits];  // left operand rows (output rows i)
  u32x4 q[2][kBN][kUnits];  // right operand rows (output columns j)
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 8 x 8 bf16 transpose: v[r] holds row r (8 columns, 2 per dword); returns
// w[c] holding column c (8 rows, 2 per dword, row 2j in the low half).
__device__ __forceinline__ void transpose8x8(const u32x4 (&v)[8], u32x4 (&w)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // low half from row 2j, high half from row 2j+1, column c
      w[c][j] = __builtin_amdgcn_perm(v[2 * j + 1][c >> 1], v[2 * j][c >> 1], sel);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ns_gemm_kernel(const uint16_t* __restrict__ in0, const uint16_t* __restrict__ in1,
                    uint16_t* __restrict__ out, int n_pad, int m_pad, int tiles_n,
                    int tiles_per_mat, float alpha, float beta) {
  __shared__ Lds lds;

  // ---- which matrix and tile
  const uint32_t bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int mat = bid / tiles_per_mat;
  const int t = bid % tiles_per_mat;
  const int ti = t / tiles_n, tj = t % tiles_n;
  const int i0 = ti * kBM, j0 = tj * kBN;

  // Left operand P (rows i, K-contiguous), right operand Q (rows j).
  const int64_t nn = static_cast<int64_t>(n_pad) * n_pad, nm = static_cast<int64_t>(n_pad) * m_pad;
  const uint16_t* P;
  const uint16_t* Q;
  int ldp, K;
  if constexpr (MODE == 0) {  // A = X X^T: P = Q = X (n_pad x m_pad)
    P = in0 + mat * nm;
    Q = P;
    ldp = m_pad;
    K = m_pad;
  } else if constexpr (MODE == 1) {  // B = b A + c A A^T: P = Q = A (n_pad x n_pad)
    P = in0 + mat * nn;
    Q = P;
    ldp = n_pad;
    K = n_pad;
  } else {  // X' = a X + B X: P = B (n_pad x n_pad), Q^T = X (n_pad x m_pad)
    P = in0 + mat * nn;
    Q = in1 + mat * nm;
    ldp = n_pad;
    K = n_pad;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> register staging
  // K-contiguous tile: thread loads unit tid%8 of rows tid/8 + 32*jj.
  const int ld_unit = tid & 7, ld_row = tid >> 3;
  // transposed tile (mode 2): k-chunk tid%8 (8 rows of X), column chunk tid/8.
  const int tr_kc = tid & 7, tr_cc = tid >> 3;

  u32x4 regP[8], regQ[8];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      regP[jj] = ld_global16(P + static_cast<int64_t>(i0 + ld_row + 32 * jj) * ldp + k0 + 8 * ld_unit);
    if constexpr (MODE != 2) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        regQ[jj] = ld_global16(Q + static_cast<int64_t>(j0 + ld_row + 32 * jj) * ldp + k0 + 8 * ld_unit);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        regQ[r] = ld_global16(Q + static_cast<int64_t>(k0 + 8 * tr_kc + r) * m_pad + j0 + 8 * tr_cc);
    }
  };

  auto store_stage = [&](int s) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int row = ld_row + 32 * jj;
      lds.p[s][row][ld_unit ^ (row & 7)] = regP[jj];
    }
    if constexpr (MODE != 2) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int row = ld_row + 32 * jj;
        lds.q[s][row][ld_unit ^ (row & 7)] = regQ[jj];
      }
    } else {
      u32x4 w[8];
      transpose8x8(regQ, w);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int row = 8 * tr_cc + c;  // row & 7 == c
        lds.q[s][row][tr_kc ^ c] = w[c];
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  const int frag_row = lane & 31, frag_half = lane >> 5, swz = lane & 7;

  auto compute_stage = [&](int s) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int unit = (2 * ks + frag_half) ^ swz;
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        fa[x] = as_bf16x8(lds.q[s][wn * 128 + x * 32 + frag_row][unit]);
        fb[x] = as_bf16x8(lds.p[s][wm * 128 + x * 32 + frag_row][unit]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
  };

  // ---- main loop: one barrier per K step
  const int KT = K / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage((kt + 1) * kBK);
    compute_stage(cur);
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: acc[x][y] holds C[i][j] for i = rows of tile y, j = rows of tile x
  const int ldo = (MODE == 2) ? m_pad : n_pad;
  uint16_t* O = out + mat * ((MODE == 2) ? nm : nn);
  const uint16_t* E = nullptr;  // epilogue operand (A for mode 1, X for mode 2)
  if constexpr (MODE == 1) E = in0 + mat * nn;
  if constexpr (MODE == 2) E = in1 + mat * nm;
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int64_t i = i0 + wm * 128 + y * 32 + frag_row;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t j = j0 + wn * 128 + x * 32 + 8 * g + 4 * frag_half;
        float v0 = acc[x][y][4 * g + 0], v1 = acc[x][y][4 * g + 1];
        float v2 = acc[x][y][4 * g + 2], v3 = acc[x][y][4 * g + 3];
        if constexpr (MODE == 1 || MODE == 2) {
          const u32x2 e = *reinterpret_cast<const u32x2*>(E + i * ldo + j);
          const float sa = alpha, sb = (MODE == 1) ? beta : 1.0f;
          v0 = sa * bf16_lo(e.x) + sb * v0;
          v1 = sa * bf16_hi(e.x) + sb * v1;
          v2 = sa * bf16_lo(e.y) + sb * v2;
          v3 = sa * bf16_hi(e.y) + sb * v3;
        }
        u32x2 o = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        *reinterpret_cast<u32x2*>(O + i * ldo + j) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_ns_gemm(int mode, const NsGeometry& g, const uint16_t* in0, const uint16_t* in1,
                          uint16_t* out, float alpha, float beta, hipStream_t stream) {
  const int n_pad = static_cast<int>(g.n_pad), m_pad = static_cast<int>(g.m_pad);
  const int tiles_m = n_pad / kBM;
  const int tiles_n = (mode == 2) ? m_pad / kBN : n_pad / kBN;
  const int tiles_per_mat = tiles_m * tiles_n;
  const int64_t blocks = static_cast<int64_t>(tiles_per_mat) * g.batch;
  dim3 grid(static_cast<unsigned>(blocks));
  switch (mode) {
    case 0:
      hipLaunchKernelGGL(ns_gemm_kernel<0>, grid, dim3(kThreads), 0, stream, in0, in1, out, n_pad,
                         m_pad, tiles_n, tiles_per_mat, alpha, beta);
      break;
    case 1:
      hipLaunchKernelGGL(ns_gemm_kernel<1>, grid, dim3(kThreads), 0, stream, in0, in1, out, n_pad,
                         m_pad, tiles_n, tiles_per_mat, alpha, beta);
      break;
    default:
      hipLaunchKernelGGL(ns_gemm_kernel<2>, grid, dim3(kThreads), 0, stream, in0, in1, out, n_pad,
                         m_pad, tiles_n, tiles_per_mat, alpha, beta);
      break;
  }
  return hipGetLastError();
}

}  // namespace mc
