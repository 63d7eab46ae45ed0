// Batched bf16 MFMA GEMMs of one Newton-Schulz step (gfx950).
//
// One step of the odd polynomial p(X) = a X + b (X X^T) X + c (X X^T)^2 X is
// three GEMMs on the zero-padded n_pad x m_pad state X:
//   mode 0  A  = Xh Xh^T                  K = m_pad   (out n_pad x n_pad)
//   mode 1  B  = b A + c A A              K = n_pad   (A symmetric: A A = A^T A)
//   mode 2  X' = a X + d Xh + N Xh        K = n_pad   (out n_pad x m_pad)
// with B split into its diagonal d (float32, one value per row) and the
// rest N (bf16, zero diagonal), so X' = a X + B Xh with B's diagonal never
// rounded.  X is carried as X = Xh + Xl: the bf16 high part and the rounding
// residual, coded in one signed byte per element as a step of the binary32
// bit pattern away from the high part's (enc_lo / dec_x in mc_device.h);
// about 16 significant bits together.  The
// products read the high part only, on v_mfma_f32_32x32x16_bf16 with float32
// accumulation; the epilogue of the third product adds a (Xh + Xl) + d Xh in
// float32 and splits X' into its two parts again.
//
// Why: along singular directions with small singular values the iteration
// acts as x -> a x (a = 3.4445), so an error there grows about a^5 ~ 490-fold
// over five steps.  Rounding X (or B' = a I + B with a folded diagonal) to
// bf16 puts an error of 2^-9 of X's largest components into every direction,
// which swamps the small ones of low-rank or decaying spectra.  With a X
// exact to 16 bits, the error left is B's rounding and the dropped B Xl, both
// along B's range (the large singular directions), where it is relatively
// small; d stays exact because a + d nearly cancels as a singular value
// converges (d -> 1 - a), which would magnify a rounded d.  A bf16 emulation
// against the exact result at 2048 x 7168, relative Frobenius error of this
// form (of the folded all-bf16 form): rank 1 2.6e-3 (1.18), rank 16 plus
// noise 2.4e-3 (0.38), four decades of singular values 4.8e-3 (3.7e-2),
// Gaussian 8.3e-3 (7.0e-3).  (Adding d Xl as well would help Gaussian
// matrices but move the dropped remainder off B's range: rank 1 at 4 x 300
// then reaches 0.3.)  A and B are symmetric, so modes 0/1 compute only the
// tiles on and above the diagonal and write each off-diagonal tile twice.
//
// Tiling: a 512-thread workgroup (8 wave64s, 2 x 4, two per SIMD) owns a
// 256 x 256 output tile; each wave owns 128 x 64 = 4 x 2 MFMA tiles of
// 32 x 32 (128 float32 accumulators per lane).  K advances 32 at a time
// through LDS stages of 32 KB (two 16 KB operand tiles each): 4 for X' = B'X,
// 5 for the symmetric products (measured fastest for each).  Two waves
// per SIMD read a third more fragment bytes from LDS than four waves of
// 128 x 128 would, but each hides the other's LDS and barrier waits behind
// its MFMAs (measured: 1-3 % faster, results bit-identical).
//
// Global -> LDS: global_load_lds_dwordx4 moves 16 bytes per lane straight into
// LDS (lane l of a wave lands at the instruction's LDS base + 16 l), so the
// next stages stream in without staging registers while the current stage's
// MFMAs run.  Because the LDS slot of each lane is fixed, the XOR swizzles
// below are applied on the global side: each lane fetches the 16 bytes that
// belong in its slot.
//
// Operand tiles.  The left tile is always K-contiguous in LDS: row r (an
// output index) holds 32 consecutive k as 4 units of 16 bytes, unit u at
// u ^ swizzle(r), read with ds_read_b128.  It comes from
//  * X itself for X X^T (X is stored in panels of 32 columns, so the tile of
//    a K-step is one contiguous 16 KB run of a panel), or
//  * A or B' for the other two products, which this file stores in a blocked
//    layout (256 x 32 blocks, row-major inside): a K-contiguous 256 x 32 tile
//    of A or B' is one contiguous 16 KB block.  A and B' are symmetric, so
//    their row panels are the column panels the products need.
// The right tile is the same kind of tile for X X^T and A A; for B' X it is a
// "K-rows" tile of X (row-major with K as its row index): 32 k-rows x 256
// output indices, the same 32 rows of eight panels (16 rows x 64 bytes, one
// contiguous 1 KB run, per DMA instruction), and fragments come from
// ds_read_b64_tr_b16, which hands
// each lane 4 consecutive k of one column (measured on gfx950: within each
// 16-lane group, lane i receives element i % 4 of the 4 x 16-bit values
// addressed by lanes i / 4 + 4 e, e = 0..3); two of them make one 8-k MFMA
// operand.  Measured on MI355X: ds_read_b128 fragments stall the MFMA
// pipeline about 2.5 x less per K step than transposed b64 reads, and a
// contiguous 1 KB DMA instruction is the fastest LDS-DMA pattern.
//
// MFMA operand roles: the MFMA "A" operand is the right-hand tile (output
// columns j) and "B" the left-hand tile (output rows i), so each lane ends up
// holding 4 consecutive j of one output row i per 4-register group and the
// epilogue reads and writes 8-byte runs.
// Lane layout of v_mfma_f32_32x32x16_bf16 (measured on gfx950): A/B lane l
// holds row/column l % 32, k = 8 * (l / 32) + [0, 8); result register r of
// lane l is row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.

#include <type_traits>

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kWaves = 8, kThreads = 64 * kWaves;  // 2 x 4 waves, 2 per SIMD
constexpr int kWaveCols = kBN / 4;                   // 64 output columns per wave
constexpr int kCT = kWaveCols / 32;                  // 32-column MFMA tiles per wave
constexpr int kMaxStages = 5;  // LDS stages in flight (prefetch distance stages - 1), per mode below
constexpr int kTileBytes = kBK * kBN * 2;  // 16 KB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kLoadsPerTile = kTileBytes / 1024 / kWaves;  // DMA instructions per wave per operand tile
constexpr int kLoadsPerStage = 2 * kLoadsPerTile;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2_t;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// K-contiguous tile: unit u of row r sits at u ^ swizzle(r).  Over 16
// consecutive rows the pair (r & 3, swizzle(r)) takes 16 distinct values, so
// a ds_read_b128 of consecutive rows at one unit touches 16 different 16-byte
// bank groups per 256 bytes.
__device__ __forceinline__ int swizzle(int r) { return (r >> 2) & 3; }


// One global_load_lds_dwordx4: 16 bytes from g_uniform + lane_off to LDS
// address m0 + 16 * lane.  Written as inline asm so the compiler's waitcnt
// insertion does not treat every later LDS read as a possible alias of the
// in-flight copy (it would otherwise wait for the copy before each read);
// completion is awaited explicitly (wait_vmem) before the barrier that
// publishes a stage.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const char* g_uniform, uint32_t lane_off, uint32_t lds_addr) {
  // the base is wave-uniform by construction; readfirstlane lets the compiler
  // keep it in SGPRs where it cannot prove that itself
  const uint64_t a = reinterpret_cast<uintptr_t>(g_uniform);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
  const char* base = reinterpret_cast<const char*>(lo | (hi << 32));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2\n"
               :
               : "s"(lds_addr), "v"(lane_off), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Per-lane byte offsets of the tile loads.  A tile is 16 pieces of 1 KB;
// wave w fills pieces c = w + 8 jj (LDS offset 1024 c, lane l at + 16 l).
// The swizzle of a lane's row does not depend on jj, so each lane has one
// offset per tile and every load is "uniform base + jj * stride + lane
// offset" (SGPR-base addressing).
//
// K-contiguous 256 x 32 tile (row pitch ld elements): piece c is rows
// 16 c .. 16 c + 15; lane l takes row 16 c + l / 4, slot l % 4, and
// swizzle(row) = (l / 16) & 3 for every jj; the stride is 128 rows.
__device__ __forceinline__ uint32_t kc_lane_offset(int64_t ld, int wave, int lane) {
  const int r = 16 * wave + (lane >> 2);
  const int u = (lane & 3) ^ ((lane >> 4) & 3);
  return static_cast<uint32_t>((r * ld + 8 * u) * 2);
}
// K-rows 32 x 256 tile of X (panels of 32 columns, x_off): piece c is rows
// 16 (c & 1) .. + 15 of the tile's panel c / 2, one contiguous 1 KB run;
// wave w's pieces are panels w / 2 + 4 jj (the stride is 4 panels), lane l
// takes row 16 (w & 1) + l / 4, 16-byte unit l % 4.  In LDS, panel b then
// sits at 2 KB b with 64-byte rows (no swizzle: the four rows a transposed
// read touches fill four different 64-byte bank slots by themselves).
__device__ __forceinline__ uint32_t kr_lane_offset(int64_t n_pad, int wave, int lane) {
  const int r = 16 * (wave & 1) + (lane >> 2);
  return static_cast<uint32_t>(((wave >> 1) * n_pad * 32 + r * 32 + 8 * (lane & 3)) * 2);
}

// Issue one operand tile (its pieces at g + jj * stride bytes + the lane
// offsets); `end` is one past the operand's last byte (checked in debug
// builds only).
__device__ __forceinline__ void issue_tile(const uint16_t* g, int64_t stride, uint32_t lane_off, uint32_t lds,
                                           int wave, const char* end) {
  const char* base = reinterpret_cast<const char*>(g);
#pragma unroll
  for (int jj = 0; jj < kLoadsPerTile; ++jj) {
    const char* src = base + jj * stride;
    if (MC_GUARD(0, src + lane_off + 16 <= end)) load_lds16(src, lane_off, lds + 1024 * (wave + kWaves * jj));
  }
}

// One of the kLoadsPerTile DMA instructions of an operand tile.
__device__ __forceinline__ void issue_tile_part(const uint16_t* g, int64_t stride, uint32_t lane_off, uint32_t lds,
                                                int wave, int jj, const char* end) {
  const char* src = reinterpret_cast<const char*>(g) + jj * stride;
  if (MC_GUARD(0, src + lane_off + 16 <= end)) load_lds16(src, lane_off, lds + 1024 * (wave + kWaves * jj));
}

// K-rows tiles: per-lane LDS read address (relative to a stage) of the
// fragment of 32-column MFMA tile x of an operand tile at tile_off, for
// k-rows 0..3; the upper four k (+256 bytes), the k sub-step (+1 KB) and
// the stage are uniform offsets.  Lane l (16-lane group g = l / 16,
// i = l % 16) addresses k-row 8 (g / 2) + i / 4 and columns
// col_base + 32 x + 16 (g & 1) + 4 (i & 3) .. + 3 (panel
// (col_base + 32 x) / 32; col_base is a multiple of 32).
constexpr int kTrHi = 4 * 64, kTrSubstep = 16 * 64;
__device__ __forceinline__ uint32_t tr_addr(int tile_off, int col_base, int x, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int r = 8 * (g >> 1) + (i >> 2);
  const int panel = (col_base + 32 * x) >> 5;
  return tile_off + panel * 2048 + r * 64 + (16 * (g & 1) + 4 * (i & 3)) * 2;
}

// Per-lane LDS read addresses relative to a stage; everything else that
// varies inside a stage is a compile-time or uniform offset.  The left tile
// is always K-contiguous (p[ks] per k16 sub-step, + 2 KB per 32-row MFMA
// tile); the right tile is K-contiguous (q[ks], modes 0/1) or K-rows (q[x]
// per 32-column MFMA tile, mode 2).
struct FragAddr {
  uint32_t p[2];
  uint32_t q[4];
};

template <bool Q_KROWS>
__device__ __forceinline__ FragAddr frag_addresses(int lane, int wm, int wn) {
  FragAddr a;
  // K-contiguous: lane l reads row l % 32 of each 32-row MFMA tile,
  // k = 8 (l / 32) + 16 ks .. + 7
  const int frag_row = lane & 31, frag_half = lane >> 5, swz = swizzle(frag_row);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int unit = (2 * ks + frag_half) ^ swz;
    a.p[ks] = (wm * 128 + frag_row) * 64 + unit * 16;
    if constexpr (!Q_KROWS) a.q[ks] = kTileBytes + (wn * kWaveCols + frag_row) * 64 + unit * 16;
  }
  if constexpr (Q_KROWS) {
#pragma unroll
    for (int x = 0; x < kCT; ++x) a.q[x] = tr_addr(kTileBytes, wn * kWaveCols, x, lane);
  } else {
    a.q[2] = a.q[3] = 0;
  }
  return a;
}

// Fragment registers of one k16 sub-step.
struct Frags {
  bf16x8 a[kCT];  // right tile (output columns): MFMA "A" operand
  bf16x8 b[4];    // left tile (output rows): MFMA "B" operand
};

__device__ __forceinline__ bf16x8 tr_frag(uint32_t addr) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)(addr));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)(addr + kTrHi));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 v = {l2.x, l2.y, h2.x, h2.y};
  return as_bf16x8(v);
}

template <bool Q_KROWS>
__device__ __forceinline__ void load_frags(const FragAddr& fadr, uint32_t stage_base, int ks, Frags& f) {
  const uint32_t pb = stage_base + fadr.p[ks];
#pragma unroll
  for (int y = 0; y < 4; ++y) f.b[y] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)(pb + y * 2048));
  if constexpr (Q_KROWS) {
#pragma unroll
    for (int x = 0; x < kCT; ++x) f.a[x] = tr_frag(stage_base + fadr.q[x] + ks * kTrSubstep);
  } else {
    const uint32_t qb = stage_base + fadr.q[ks];
#pragma unroll
    for (int x = 0; x < kCT; ++x) f.a[x] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)(qb + x * 2048));
  }
}

// Part g of a sub-step's fragments: left tiles y = 2 g, 2 g + 1 and right
// tile x = g.
template <bool Q_KROWS>
__device__ __forceinline__ void load_frags_part(const FragAddr& fadr, uint32_t stage_base, int ks, int g,
                                                Frags& f) {
#pragma unroll
  for (int y = 2 * g; y < 2 * g + 2; ++y)
    f.b[y] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)(stage_base + fadr.p[ks] + y * 2048));
  if constexpr (Q_KROWS) f.a[g] = tr_frag(stage_base + fadr.q[g] + ks * kTrSubstep);
  else f.a[g] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)(stage_base + fadr.q[ks] + g * 2048));
}

// The 4 MFMAs of right tile x = g.
__device__ __forceinline__ void mfma_4(const Frags& f, int g, f32x16 (&acc)[kCT][4]) {
#pragma unroll
  for (int y = 0; y < 4; ++y) acc[g][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[g], f.b[y], acc[g][y], 0, 0, 0);
}

// Blocked layout of the n_pad x n_pad matrices A and B' (internal to a call):
// 256 x 32 blocks, row-major inside, block (r / 256, c / 32) at element
// ((r / 256) * nkb + c / 32) * 8192 with nkb = n_pad / 32.  A K-contiguous
// 256 x 32 operand tile of A or B' (rows r0.., k-block kb) is then one
// contiguous 16 KB block, which the LDS DMA reads fastest.
__device__ __forceinline__ int64_t blk_off(int r, int c, int nkb) {
  return (static_cast<int64_t>(r >> 8) * nkb + (c >> 5)) * 8192 + (r & 255) * 32 + (c & 31);
}

// Mirrored store of a symmetric result: a staged 128 x 128 bf16 region (row
// ii at eb + ii * 256, 16-byte unit u at position u ^ (ii & 15)) is written
// transposed: element (ii, jj) goes to row r0d + jj, column c0d + ii; each of
// the region's two waves runs 16 of the 32 instructions, from s_begin.
// Instruction s covers columns C = 16 (s % 8) .. + 15: 16-lane group g takes
// rows ii = R .. R + 7 with R = 64 (s / 16) + 32 (s / 8 % 2) + 8 g, lane i
// column C + i, which it assembles from two transposed reads of 4 rows each;
// so one instruction writes 16 destination rows x 64 bytes (a whole row of a
// 32-column block of the blocked layout) rather than 64 rows x 16 bytes
// (measured: X X^T 2 %, A A 4 % faster).
// dst is the matrix base; (r0, c0) the destination of staged element (0, 0)
// after the transposition; the destination is blocked.
__device__ __forceinline__ void store_transposed(uint32_t eb, uint16_t* dst, int r0d, int c0d, int nkb, int lane,
                                                 int s_begin) {
  const int g = lane >> 4, i = lane & 15;
#pragma unroll 4
  for (int s = s_begin; s < s_begin + 16; ++s) {
    const int R = 64 * (s >> 4) + 32 * ((s >> 3) & 1) + 8 * g, C = 16 * (s & 7);
    const int col = C + 4 * (i & 3);
    const int r0 = R + (i >> 2), r1 = r0 + 4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(uintptr_t)(eb + r0 * 256 + (((col >> 3) ^ (r0 & 15)) << 4) + (col & 7) * 2));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(uintptr_t)(eb + r1 * 256 + (((col >> 3) ^ (r1 & 15)) << 4) + (col & 7) * 2));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 v = {l2.x, l2.y, h2.x, h2.y};
    const int64_t o = blk_off(r0d + C + i, c0d + R, nkb);
    if (MC_GUARD(3, o + 8 <= static_cast<int64_t>(nkb) * 32 * nkb * 32)) *reinterpret_cast<u32x4*>(dst + o) = v;
  }
}

// Fused in-place update of the last step (mode 2): W is n x m (or m x n when
// transposed, i.e. the matrix was iterated on as its transpose).
struct UpdArgs {
  void* W;
  int64_t w_stride;  // elements between matrices
  int n, m;          // logical X shape
  float out_scale, lr, wd;
};

// UPD: 0 = store X' (or A, B'); 1 = update bf16 W; 2 = update float32 W;
// 3 / 4 = write O = out_scale * X' (transposed back for a matrix iterated on
// as its transpose) to a bf16 / float32 W, which is then the output.
// SCALED: the launch carries 1 / ||M|| per matrix (the first Newton-Schulz
// step); otherwise the epilogue has no multiply.  TR (UPD != 0 only): W is
// the transpose of X' (a matrix iterated on as its transpose); a template
// parameter so each epilogue is compiled for its own access pattern.
// Mode 1: B = alpha A + beta A A, its diagonal written to dg (float32,
// n_pad per matrix) and zero in `out`.  Mode 2 reads X's low part xl (with
// in1 = Xh) and B's diagonal dg and, unless UPD, writes X''s low part to
// xl_out; acoef is a.
template <int MODE, int UPD, bool SCALED, bool TR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_gemm_kernel(const uint16_t* __restrict__ in0, const uint16_t* __restrict__ in1,
                    const uint8_t* __restrict__ xl, uint16_t* __restrict__ out, uint8_t* __restrict__ xl_out,
                    float* __restrict__ dg, int n_pad, int m_pad, int tiles_n, int tiles_per_mat, float alpha,
                    float beta, float acoef, const float* __restrict__ inv, UpdArgs ua) {
  static_assert(UPD == 0 || MODE == 2, "only X' = B' X can apply the update");
  static_assert(UPD != 0 || !TR, "TR describes W");
  constexpr bool kQKRows = MODE == 2;      // right operand X as K-rows tiles
  constexpr bool kBlockedOut = MODE != 2;  // A, B' results in the blocked layout
  // X' = B'X runs fastest with 4 stages, the symmetric products with 5
  constexpr int kStages = MODE == 2 ? 4 : kMaxStages;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  // The epilogue reuses the stages' LDS: four 32 KB regions of the bf16
  // tile, half of it in float32 (the row-ordered epilogue), or X's parts for
  // the transposed update (96 KB).  Fewer stages would silently drop writes.
  static_assert(kStages * kStageBytes >= 4 * 32768, "the epilogue stages 128 KB in the stages' LDS");
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));

  // ---- which matrix and tile.  Modes 0/1: the upper triangle (ti <= tj),
  // row-major.  Mode 2: column-major, so tiles resident together on one XCD
  // share X panels (and all of B's few panels) in that XCD's L2.
  const uint32_t bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int mat = bid / tiles_per_mat;
  int t = bid % tiles_per_mat;
  int ti, tj;
  if constexpr (MODE == 2) {
    const int tiles_m = n_pad / kBM;
    ti = t % tiles_m;
    tj = t / tiles_m;
  } else {
    ti = 0;
    while (t >= tiles_n - ti) {
      t -= tiles_n - ti;
      ++ti;
    }
    tj = ti + t;
  }
  const int i0 = ti * kBM, j0 = tj * kBN;

  const int64_t nn = static_cast<int64_t>(n_pad) * n_pad, nm = static_cast<int64_t>(n_pad) * m_pad;
  const int nkb = n_pad / kBK;  // k-blocks per row of the blocked layout
  // Operand tiles at k = 0, their row pitch (K-contiguous tiles), the byte
  // stride between a wave's two DMA pieces and the element step between
  // K-steps (X in panels of 32 columns, see x_off; A and B' blocked).
  //   mode 0: rows i0.. and j0.. of X, K-contiguous: K-step kt is panel kt,
  //           one contiguous 16 KB run
  //   mode 1: blocks of A at rows i0.. and j0.. (pitch 32, step one block)
  //   mode 2: blocks of B' at rows i0.. (symmetric: rows are columns), and
  //           k-rows 32 kt.. of X's panels j0 / 32 .. j0 / 32 + 7: eight
  //           contiguous 2 KB runs
  const int64_t panel = static_cast<int64_t>(n_pad) * 32;
  const uint16_t* Pg;
  const uint16_t* Qg;
  int64_t ldp, ldq, kstep_p, kstep_q, jstride_p, jstride_q;
  int K;
  if constexpr (MODE == 0) {
    Pg = in0 + mat * nm + static_cast<int64_t>(i0) * 32;
    Qg = in0 + mat * nm + static_cast<int64_t>(j0) * 32;
    ldp = ldq = 32;
    kstep_p = kstep_q = panel;
    jstride_p = jstride_q = 128 * 32 * 2;
    K = m_pad;
  } else if constexpr (MODE == 1) {
    Pg = in0 + mat * nn + blk_off(i0, 0, nkb);
    Qg = in0 + mat * nn + blk_off(j0, 0, nkb);
    ldp = ldq = kBK;
    kstep_p = kstep_q = kBM * kBK;
    jstride_p = jstride_q = 128 * kBK * 2;
    K = n_pad;
  } else {
    Pg = in0 + mat * nn + blk_off(i0, 0, nkb);
    Qg = in1 + mat * nm + x_off(0, j0, n_pad);
    ldp = kBK;
    kstep_p = kBM * kBK;
    jstride_p = 128 * kBK * 2;
    ldq = n_pad;  // kr_lane_offset takes the panel height
    kstep_q = kBK * 32;
    jstride_q = 4 * panel * 2;
    K = n_pad;
  }
  // one past each operand (range checks of debug builds): in0 holds X (mode
  // 0), A or B' (modes 1, 2); in1 holds X (mode 2)
  const int64_t nmat = gridDim.x / tiles_per_mat;
  const char* const end_p = reinterpret_cast<const char*>(in0 + nmat * (MODE == 0 ? nm : nn));
  const char* const end_q = MODE == 2 ? reinterpret_cast<const char*>(in1 + nmat * nm) : end_p;
  // element offset of K-step kt from the operand origin
  auto k_ofs = [&](int kt, int64_t kstep) -> int64_t { return kt * kstep; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  const uint32_t off_p = kc_lane_offset(ldp, wave, lane);
  const uint32_t off_q = kQKRows ? kr_lane_offset(ldq, wave, lane) : kc_lane_offset(ldq, wave, lane);
  const int KT = K / kBK;
  // Loads of K-step kt into stage kt % kStages.  Past the last step the last
  // in-bounds tile is fetched again into a stage nobody reads, which keeps
  // the number of loads in flight (and so the wait counts) fixed.
  auto issue_p = [&](int kt) {
    issue_tile(Pg + k_ofs(min(kt, KT - 1), kstep_p), jstride_p, off_p, lds + (kt % kStages) * kStageBytes, wave,
                      end_p);
  };
  auto issue_q = [&](int kt) {
    issue_tile(Qg + k_ofs(min(kt, KT - 1), kstep_q), jstride_q, off_q,
                        lds + (kt % kStages) * kStageBytes + kTileBytes, wave, end_q);
  };
  const FragAddr fadr = frag_addresses<kQKRows>(lane, wm, wn);

  f32x16 acc[kCT][4];
#pragma unroll
  for (int a = 0; a < kCT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  // ---- main loop: kStages - 1 K-steps in flight.  At step kt the stage of
  // kt + kStages - 1 is refilled (it was last read at step kt - 1, before the
  // barrier) in two halves, one per half step, so no wave blocks on a burst of
  // copies; stage kt is consumed; the mid-step wait leaves only newer loads
  // outstanding, so step kt + 1 is complete.  The two k16 sub-steps of a
  // step are software-pipelined across the barrier: sub-step 1's fragments
  // load under sub-step 0's MFMAs, and the next step's sub-step 0 fragments
  // load under sub-step 1's MFMAs.
  for (int s = 0; s < kStages - 1; ++s) {
    issue_p(s);
    issue_q(s);
  }
  wait_vmem<(kStages - 2) * kLoadsPerStage>();
  __syncthreads();
  Frags f0, f1;
  load_frags<kQKRows>(fadr, lds, 0, f0);
  // One half step: the 8 MFMAs of fragments fc in kCT = 2 groups (right tile
  // x = g), each preceded by one DMA instruction of the refill and followed
  // by part g of the next sub-step's fragment reads into fn, with a
  // scheduling fence after each group, so copies and reads stay spread over
  // the half step instead of bunching up (a DMA instruction the memory
  // pipeline cannot take yet stalls the in-order issue of everything behind
  // it).  Inside a group the scheduler orders MFMAs and reads itself.
  // Measured against the unfenced groups: B'X 3-5 %, A A 7-9 %, X X^T 2-3 %
  // faster.
  auto half = [&](const Frags& fc, Frags& fn, uint32_t rd_stage, int rd_ks, auto&& dma) {
#pragma unroll
    for (int g = 0; g < kCT; ++g) {
      dma(g);
      mfma_4(fc, g, acc);
      load_frags_part<kQKRows>(fadr, rd_stage, rd_ks, g, fn);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < KT; ++kt) {
    const uint32_t cur = lds + (kt % kStages) * kStageBytes;
    const uint32_t nxt = lds + ((kt + 1) % kStages) * kStageBytes;
    const int kr = min(kt + kStages - 1, KT - 1);
    const uint32_t refill = lds + ((kt + kStages - 1) % kStages) * kStageBytes;
    half(f0, f1, cur, 1, [&](int jj) {
      issue_tile_part(Pg + k_ofs(kr, kstep_p), jstride_p, off_p, refill, wave, jj, end_p);
    });
    wait_vmem<(kStages - 2) * kLoadsPerStage - kLoadsPerTile>();
    __syncthreads();
    // After the last step this reads a stage of redundant tiles; unused.
    half(f1, f0, nxt, 0, [&](int jj) {
      issue_tile_part(Qg + k_ofs(kr, kstep_q), jstride_q, off_q, refill + kTileBytes, wave, jj, end_q);
    });
  }

  // ---- epilogue, staged through LDS (free once every stage is consumed).
  // The tile is staged as four 128 x 128 regions (rows i0 + 128 wm, columns
  // j0 + 128 (wn / 2)), region k at lds + 32 KB k: row ii at ii * 256 bytes,
  // 16-byte unit u at position u ^ (ii & 15); the two waves of a region each
  // write their 64 columns and then take half of its rows of global traffic,
  // which is whole 256-byte rows:
  //   mode 1: every lane combines its accumulators with the A values at
  //   their positions, b A + c (A A) (+ a on the diagonal);
  //   modes 0/2: every lane rounds its accumulators into place;
  //   the region is stored row by row, 16 bytes per lane;
  //   modes 0/1, off-diagonal tiles: it is also stored mirrored.
  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int wh = wn & 1;  // which half of the region's columns, and of its passes
  const int i0w = i0 + wm * 128, j0w = j0 + (wn >> 1) * 128;
  // X is inv_b times the stored X in the first step of the fused path
  const float xs = (inv != nullptr) ? inv[mat] : 1.0f;

  // Mode 2, update of a transposed W (the other launches take the
  // row-ordered epilogue, kRowEpi below): X' = a (Xh + Xl) + d Xh + N Xh is
  // formed in the accumulators before they are staged in bf16 for the
  // transposed update, the diagonal terms in float32 from both parts of X at
  // this lane's accumulator positions (4 consecutive columns per MFMA
  // register group).  X is brought into LDS first, half of the tile's rows
  // at a time (tile rows 128 wm + 32 (yh + yy) + r: 128 rows, 64 KB of high
  // parts and 32 KB of codes), by DMA into 512-byte (256-byte) LDS rows,
  // 16-byte unit u of LDS row lr at u ^ (lr & 31) (codes: u ^ (lr & 15)),
  // the swizzle applied on the global side (in X's panels of 32 columns a
  // row of the tile is eight 64-byte runs); each lane then reads its values
  // from LDS.  Loading them from global memory at the accumulator positions
  // instead touched 32 rows x 16 bytes per instruction (4.31 ms per
  // 64-matrix launch against 3.64 for the straight update).
  constexpr bool kRowEpi = MODE == 2 && !(UPD != 0 && TR);
  if constexpr (MODE == 2 && !kRowEpi) {
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2_t;
    typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
    constexpr uint32_t kCodes = 65536;  // LDS offset of the codes
    float dgr[4];  // d_i of this lane's 4 rows (the factor of Xh; a multiplies X)
#pragma unroll
    for (int y = 0; y < 4; ++y)
      dgr[y] = MC_GUARD(4, i0w + y * 32 + frag_row < n_pad) ? dg[static_cast<int64_t>(mat) * n_pad + i0w + y * 32 + frag_row]
                                                             : 0.f;
    // every copy of the K loop has landed and every wave is past its reads
    wait_vmem<0>();
    __syncthreads();
    const char* const xh_tile = reinterpret_cast<const char*>(in1 + mat * nm + x_off(i0, j0, n_pad));
    const char* const xl_tile = reinterpret_cast<const char*>(xl + mat * nm + x_off(i0, j0, n_pad));
    [[maybe_unused]] const char* const xh_end = reinterpret_cast<const char*>(in1 + (mat + 1) * nm);
    [[maybe_unused]] const char* const xl_end = reinterpret_cast<const char*>(xl + (mat + 1) * nm);
    // element offset of tile element (R, C) from the tile's origin (x_off)
    auto toff = [&](int R, int C) -> int64_t { return (C >> 5) * static_cast<int64_t>(n_pad) * 32 + R * 32 + (C & 31); };
#pragma unroll
    for (int yh = 0; yh < 4; yh += 2) {
      // LDS row lr = 64 wm' + 32 yy + r holds tile row 128 wm' + 32 (yh + yy) + r
      auto tile_row = [&](int lr) { return 128 * (lr >> 6) + 32 * yh + (lr & 63); };
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // high parts: 64 instructions of 1 KB, 8 per wave
        const int sl = (8 * wave + k) * 64 + lane, lr = sl >> 5, pu = sl & 31;
        const uint32_t off = static_cast<uint32_t>(2 * toff(tile_row(lr), 8 * (pu ^ (lr & 31))));
        if (MC_GUARD(6, xh_tile + off + 16 <= xh_end)) load_lds16(xh_tile, off, lds + (8 * wave + k) * 1024);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // codes: 32 instructions, 4 per wave
        const int sl = (4 * wave + k) * 64 + lane, lr = sl >> 4, pu = sl & 15;
        const uint32_t off = static_cast<uint32_t>(toff(tile_row(lr), 16 * (pu ^ (lr & 15))));
        if (MC_GUARD(6, xl_tile + off + 16 <= xl_end))
          load_lds16(xl_tile, off, lds + kCodes + (4 * wave + k) * 1024);
      }
      wait_vmem<0>();
      __syncthreads();
#pragma unroll
      for (int yy = 0; yy < 2; ++yy)
#pragma unroll
        for (int x = 0; x < kCT; ++x)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int lr = 64 * wm + 32 * yy + frag_row;
            const int c = kWaveCols * wn + 32 * x + 8 * g + 4 * frag_half;  // tile column
            const u32x2 h =
                *(const lds_u32x2_t*)(uintptr_t)(lds + lr * 512 + 16 * ((c >> 3) ^ (lr & 31)) + (c & 7) * 2);
            const uint32_t l =
                *(const lds_u32_t*)(uintptr_t)(lds + kCodes + lr * 256 + 16 * ((c >> 4) ^ (lr & 15)) + (c & 15));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t hs = hi_bits(q < 2 ? h.x : h.y, q & 1);
              acc[x][yh + yy][4 * g + q] += dgr[yh + yy] * __uint_as_float(hs) + acoef * dec_x(i8_at(l, q), hs);
            }
          }
      // the next half's copies (or the staging) reuse the LDS
      __syncthreads();
    }
  }
  wait_vmem<0>();
  __syncthreads();

  // Mode 2, row-ordered epilogue: the accumulators are staged in float32,
  // half of the tile (256 rows x 128 columns, 128 KB) at a time, by the four
  // waves that own those columns; then every lane takes 8 consecutive
  // columns of a row per pass (16 lanes per row, 4 consecutive rows per
  // wave), reads X's two parts there with 16-byte loads (a wave's 64 lanes
  // cover 256 contiguous bytes of each of 4 panels of 32 columns), forms
  // X' = xs (a (Xh + Xl) + d_i Xh + N Xh) in float32 and writes X''s two
  // parts, or
  // applies the update / writes the output, with 16-byte accesses.  Staged
  // row r holds 16-byte unit u (4 columns) at u ^ (r & 31).
  if constexpr (kRowEpi) {
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
    const uint16_t* Xh = in1 + mat * nm;
    const uint8_t* Xlm = xl + mat * nm;
    const float* dgm = dg + static_cast<int64_t>(mat) * n_pad;
    auto fst = [&](int r, int u) -> uint32_t { return lds + r * 512 + ((u ^ (r & 31)) << 4); };
    const int cg = tid & 15, rsub = tid >> 4;
    constexpr bool kReadW = UPD == 1 || UPD == 2;
    constexpr int kEsz = (UPD == 2 || UPD == 4) ? 4 : 2;
    constexpr int kWords = (UPD == 2 || UPD == 4) ? 2 : 1;  // 16-byte words per 8 elements of W
    char* const Wb = UPD != 0 ? static_cast<char*>(ua.W) + static_cast<int64_t>(mat) * ua.w_stride * kEsz : nullptr;
    const bool wvec = UPD != 0 && ua.m % 8 == 0 && reinterpret_cast<uintptr_t>(Wb) % 16 == 0;
    // X's two parts for the lane's 16 passes (8 per half, s = 8 h + p) in a
    // ring of kRing (4; 2 for float32 W, whose loads take the registers):
    // the first kRing are loaded before the staging (their latency overlaps
    // it), pass s + kRing as pass s is consumed.  a + d_i per pass row.
    constexpr int kRing = UPD == 2 ? 2 : 4;
    u32x4 xhv[kRing];
    u32x2 xlv[kRing];
    float dgr[8];
    // Non-temporal loads: each X element is read here once, and at the
    // default cache policy these 196 KB per tile evict from the XCD's L2 the
    // operand panels that the other tiles' K loops share (measured: the
    // launch 1.2-1.4 % faster, results bit-identical).
    auto load_x = [&](int sq) {
      const int64_t off = x_off(i0 + (sq & 7) * 32 + rsub, j0 + 128 * (sq >> 3) + 8 * cg, n_pad);
      if (MC_GUARD(5, off + 8 <= nm)) {
        xhv[sq % kRing] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Xh + off));
        xlv[sq % kRing] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(Xlm + off));
      } else {
        xhv[sq % kRing] = u32x4{0u, 0u, 0u, 0u};
        xlv[sq % kRing] = u32x2{0u, 0u};
      }
    };
#pragma unroll
    for (int sq = 0; sq < kRing; ++sq) load_x(sq);
#pragma unroll
    for (int p = 0; p < 8; ++p) dgr[p] = MC_GUARD(4, i0 + p * 32 + rsub < n_pad) ? dgm[i0 + p * 32 + rsub] : 0.f;
    // W of the update, read in batches of kWB passes
    constexpr int kWB = UPD == 2 ? 2 : (UPD == 1 ? 2 : 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((wn >> 1) == h) {
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
          for (int x = 0; x < kCT; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int r = wm * 128 + y * 32 + frag_row, u = 16 * wh + 8 * x + 2 * g + frag_half;
              *(lds_f32x4_t*)(uintptr_t)fst(r, u) =
                  f32x4{acc[x][y][4 * g + 0], acc[x][y][4 * g + 1], acc[x][y][4 * g + 2], acc[x][y][4 * g + 3]};
            }
      }
      __syncthreads();
      const int jc = j0 + 128 * h + 8 * cg;  // first column of this lane's run
#pragma unroll
      for (int p0 = 0; p0 < 8; p0 += kWB) {
        u32x4 wv[kReadW ? kWB : 1][kWords];
        if constexpr (kReadW) {
#pragma unroll
          for (int q = 0; q < kWB; ++q) {
            const int row = i0 + (p0 + q) * 32 + rsub;
            if (wvec && row < ua.n && jc + 8 <= ua.m &&
                MC_GUARD(2, static_cast<int64_t>(row) * ua.m + jc + 8 <= static_cast<int64_t>(ua.n) * ua.m)) {
              const u32x4* pw = reinterpret_cast<const u32x4*>(Wb + (static_cast<int64_t>(row) * ua.m + jc) * kEsz);
#pragma unroll
              for (int w = 0; w < kWords; ++w) wv[q][w] = pw[w];
            }
          }
        }
#pragma unroll
        for (int q = 0; q < kWB; ++q) {
          const int p = p0 + q, r = p * 32 + rsub, row = i0 + r;
          const f32x4 a0 = *(const lds_f32x4_t*)(uintptr_t)fst(r, 2 * cg);
          const f32x4 a1 = *(const lds_f32x4_t*)(uintptr_t)fst(r, 2 * cg + 1);
          const int sq = 8 * h + p;
          const u32x4 hq = xhv[sq % kRing];
          const u32x2 lq = xlv[sq % kRing];
          const uint32_t hw[4] = {hq.x, hq.y, hq.z, hq.w};
          float hv[8], xv[8];  // Xh and X = Xh + Xl
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t hs = hi_bits(hw[e >> 1], e & 1);
            hv[e] = __uint_as_float(hs);
            xv[e] = dec_x(i8_at(e < 4 ? lq.x : lq.y, e & 3), hs);
          }
          if (sq + kRing < 16) load_x(sq + kRing);
          const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] = av[e] + dgr[p] * hv[e] + acoef * xv[e];
            if constexpr (SCALED) v[e] *= xs;
          }
          if constexpr (UPD == 0) {
            const u32x4 ho = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                              pack_bf16x2(v[6], v[7])};
            const uint32_t ow[4] = {ho.x, ho.y, ho.z, ho.w};
            int32_t qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = enc_lo(v[e], hi_bits(ow[e >> 1], e & 1));
            const int64_t off = x_off(row, jc, n_pad);
            if (MC_GUARD(1, off + 8 <= nm)) {
              *reinterpret_cast<u32x4*>(out + mat * nm + off) = ho;
              *reinterpret_cast<u32x2*>(xl_out + mat * nm + off) =
                  u32x2{pack_i8x4(qv[0], qv[1], qv[2], qv[3]), pack_i8x4(qv[4], qv[5], qv[6], qv[7])};
            }
          } else {
            // the last step: X' rounded to bf16, then O = out_scale X'
            if (row >= ua.n || jc >= ua.m) continue;
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = ua.out_scale * bf16_to_f32(f32_to_bf16(v[e]));
            const int64_t idx = static_cast<int64_t>(row) * ua.m + jc;
            if (!MC_GUARD(2, idx + min(8, ua.m - jc) <= static_cast<int64_t>(ua.n) * ua.m)) continue;
            if (wvec && jc + 8 <= ua.m) {
              u32x4* pw = reinterpret_cast<u32x4*>(Wb + idx * kEsz);
              if constexpr (UPD == 3) {
                pw[0] = u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])};
              } else if constexpr (UPD == 4) {
                pw[0] = __builtin_bit_cast(u32x4, f32x4{o[0], o[1], o[2], o[3]});
                pw[1] = __builtin_bit_cast(u32x4, f32x4{o[4], o[5], o[6], o[7]});
              } else if constexpr (UPD == 1) {
                u32x4 w = wv[q][0];
                w.x = pack_bf16x2(update_op(bf16_lo(w.x), o[0], ua.lr, ua.wd), update_op(bf16_hi(w.x), o[1], ua.lr, ua.wd));
                w.y = pack_bf16x2(update_op(bf16_lo(w.y), o[2], ua.lr, ua.wd), update_op(bf16_hi(w.y), o[3], ua.lr, ua.wd));
                w.z = pack_bf16x2(update_op(bf16_lo(w.z), o[4], ua.lr, ua.wd), update_op(bf16_hi(w.z), o[5], ua.lr, ua.wd));
                w.w = pack_bf16x2(update_op(bf16_lo(w.w), o[6], ua.lr, ua.wd), update_op(bf16_hi(w.w), o[7], ua.lr, ua.wd));
                pw[0] = w;
              } else {
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                  f32x4 t = __builtin_bit_cast(f32x4, wv[q][w]);
                  t.x = update_op(t.x, o[4 * w + 0], ua.lr, ua.wd);
                  t.y = update_op(t.y, o[4 * w + 1], ua.lr, ua.wd);
                  t.z = update_op(t.z, o[4 * w + 2], ua.lr, ua.wd);
                  t.w = update_op(t.w, o[4 * w + 3], ua.lr, ua.wd);
                  pw[w] = __builtin_bit_cast(u32x4, t);
                }
              }
            } else {
              const int valid = min(8, ua.m - jc);
              for (int e = 0; e < valid; ++e) {
                if constexpr (UPD == 3) {
                  reinterpret_cast<uint16_t*>(Wb)[idx + e] = f32_to_bf16(o[e]);
                } else if constexpr (UPD == 4) {
                  reinterpret_cast<float*>(Wb)[idx + e] = o[e];
                } else if constexpr (UPD == 1) {
                  uint16_t* pw = reinterpret_cast<uint16_t*>(Wb) + idx + e;
                  *pw = f32_to_bf16(update_op(bf16_to_f32(*pw), o[e], ua.lr, ua.wd));
                } else {
                  float* pw = reinterpret_cast<float*>(Wb) + idx + e;
                  *pw = update_op(*pw, o[e], ua.lr, ua.wd);
                }
              }
            }
          }
        }
      }
      // the next half reuses the staging
      __syncthreads();
    }
    return;
  }

  uint16_t* O = out + mat * ((MODE == 2) ? nm : nn);
  const uint32_t eb = lds + (2 * wm + (wn >> 1)) * 32768;
  auto st_addr = [&](int ii, int u) -> uint32_t { return eb + ii * 256 + ((u ^ (ii & 15)) << 4); };

  // Fused update (UPD != 0): this wave's 16 passes of W are loaded after the
  // accumulators are staged (loading bf16 W before the staging overlapped
  // its latency, 6 % faster without the linear-term fold, but W, the fold's
  // X values and the accumulators no longer fit in the registers together).
  // Pass s:
  // straight W, lane takes staged row 4 s + lane / 16, unit lane % 16 (W row
  // i0w + row, 8 columns); transposed W, lane takes staged column
  // jj = C + lane % 16 and rows R .. R + 7 (two transposed reads), i.e. 8
  // consecutive elements of W row j0w + jj, with C = 16 (s % 8) and
  // R = 64 (s / 16) + 32 (s / 8 % 2) + 8 (lane / 16): the four 16-lane
  // groups take the same 16 W rows and 32 consecutive columns, so an
  // instruction touches 16 rows x 64 bytes of W rather than 64 rows x 16.
  constexpr bool kReadW = UPD == 1 || UPD == 2;  // 3 / 4 only write
  constexpr int kEsz = (UPD == 2 || UPD == 4) ? 4 : 2;
  constexpr int kWords = (UPD == 2 || UPD == 4) ? 2 : 1;  // 16-byte words per 8 elements
  const int ug = lane >> 4, uil = lane & 15;
  char* const Wb = UPD != 0 ? static_cast<char*>(ua.W) + static_cast<int64_t>(mat) * ua.w_stride * kEsz : nullptr;
  const int64_t wcols = TR ? ua.n : ua.m;
  const bool wvec = wcols % 8 == 0 && reinterpret_cast<uintptr_t>(Wb) % 16 == 0;
  auto pos = [&](int s, int64_t& wrow, int64_t& wcol, int& valid) {
    if constexpr (!TR) {
      const int row = 4 * s + ug;
      wrow = i0w + row;
      wcol = j0w + 8 * uil;
      valid = wrow < ua.n ? min(8, ua.m - static_cast<int>(wcol)) : 0;
    } else {
      const int R = 64 * (s >> 4) + 32 * ((s >> 3) & 1) + 8 * ug, C = 16 * (s & 7);
      wrow = j0w + C + uil;
      wcol = i0w + R;
      valid = wrow < ua.m ? min(8, ua.n - static_cast<int>(wcol)) : 0;
    }
  };
  u32x4 wbuf[kReadW ? 16 : 1][kWords];
  // W's 16 vector runs of this wave (UPD 1 / 2 only; wbuf has one slot otherwise)
  auto load_w = [&]() {
    if constexpr (kReadW) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int64_t wrow, wcol;
        int valid;
        pos(16 * wh + e, wrow, wcol, valid);
        if (wvec && valid == 8 && MC_GUARD(2, wrow * wcols + wcol + 8 <= static_cast<int64_t>(ua.n) * ua.m)) {
          const u32x4* p = reinterpret_cast<const u32x4*>(Wb + (wrow * wcols + wcol) * kEsz);
#pragma unroll
          for (int w = 0; w < kWords; ++w) wbuf[e][w] = p[w];
        }
      }
    }
  };

  // mode 1: the A values at this lane's accumulator positions (4 consecutive
  // columns, 8 bytes of the blocked layout, per MFMA register group), loaded
  // into registers before the staging so their latency overlaps it
  u32x2 abuf[MODE == 1 ? 4 : 1][MODE == 1 ? kCT : 1][MODE == 1 ? 4 : 1];
  if constexpr (MODE == 1) {
    const uint16_t* Am = in0 + mat * nn;
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int x = 0; x < kCT; ++x)
#pragma unroll
        for (int g = 0; g < 4; ++g)
        {
          const int64_t o = blk_off(i0w + y * 32 + frag_row, j0w + kWaveCols * wh + 32 * x + 8 * g + 4 * frag_half, nkb);
          abuf[y][x][g] = MC_GUARD(5, o + 4 <= nn) ? *reinterpret_cast<const u32x2*>(Am + o) : u32x2{0u, 0u};
        }
  }
  // the region straddles B's diagonal (mode 1)
  const bool on_diag = MODE == 1 && i0w == j0w;
  // The value of accumulator group (y, x, g) as the epilogue rounds it:
  // scaled by 1/||M|| in the first step, combined with A in mode 1.
  auto value = [&](int y, int x, int g, float (&v)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = acc[x][y][4 * g + q];
    if constexpr (MODE == 0 && SCALED) {
      const float s2 = xs * xs;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] *= s2;
    } else if constexpr (MODE == 2 && SCALED) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] *= xs;
    }
    if constexpr (MODE == 1) {
      const u32x2 e = abuf[y][x][g];
      const float ev[4] = {bf16_lo(e.x), bf16_hi(e.x), bf16_lo(e.y), bf16_hi(e.y)};
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = alpha * ev[q] + beta * v[q];
      // the diagonal leaves the bf16 matrix for dg (float32)
      if (on_diag) {
        const int ii = y * 32 + frag_row, jj0 = kWaveCols * wh + 32 * x + 8 * g + 4 * frag_half;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (ii == jj0 + q) {
            if (MC_GUARD(4, i0w + ii < n_pad)) dg[static_cast<int64_t>(mat) * n_pad + i0w + ii] = v[q];
            v[q] = 0.f;
          }
      }
    }
  };
  // Stage the bf16 values (modes 0/1, and mode 2 for a transposed W's update).
  auto stage = [&]() {
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int ii = y * 32 + frag_row;
#pragma unroll
      for (int x = 0; x < kCT; ++x) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t a = st_addr(ii, 8 * wh + 4 * x + g) + 8 * frag_half;
          float v[4];
          value(y, x, g, v);
          const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(lds_u32x2_t*)(uintptr_t)a = o;
        }
      }
    }
  };
  stage();
  // the region is complete once both of its waves have written
  __syncthreads();
  if constexpr (UPD != 0) {
    // Fused update instead of storing X': W <- W - lr * (out_scale * X' + wd * W)
    // (UPD 1 / 2), or the output W = out_scale * X' (UPD 3 / 4), with X'
    // rounded to bf16 as between steps; W is n x m, or m x n for a matrix
    // iterated on as its transpose.  Each lane handles 8 elements of
    // one W row per pass: 16-byte accesses, 256-byte row segments per 16
    // lanes (straight) or the mirrored-store pattern (transposed); runs that
    // leave the matrix (padding) or are misaligned go element by element.
    const bool vec = wvec;
    auto unpack8 = [](u32x4 v, float (&x)[8]) {
      x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
      x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    };
    const int g = ug, il = uil;
    auto read_x = [&](int s, float (&x)[8]) {
      if constexpr (!TR) {
        unpack8(*(const lds_u32x4_t*)(uintptr_t)st_addr(4 * s + g, il), x);
      } else {
        const int R = 64 * (s >> 4) + 32 * ((s >> 3) & 1) + 8 * g, C = 16 * (s & 7);
        const int col = C + 4 * (il & 3);
        const int r0 = R + (il >> 2), r1 = r0 + 4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(uintptr_t)(eb + r0 * 256 + (((col >> 3) ^ (r0 & 15)) << 4) + (col & 7) * 2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(uintptr_t)(eb + r1 * 256 + (((col >> 3) ^ (r1 & 15)) << 4) + (col & 7) * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        unpack8(u32x4{l2.x, l2.y, h2.x, h2.y}, x);
      }
    };
    // the wave's 16 passes
    if constexpr (kReadW) load_w();
    constexpr int kBatch = 16;
    for (int s0 = 16 * wh; s0 < 16 * wh + 16; s0 += kBatch) {
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        int64_t wrow, wcol;
        int valid;
        pos(s0 + e, wrow, wcol, valid);
        // read with every lane active: a transposed read hands each lane data
        // addressed by other lanes, which an inactive lane does not provide
        float x[8], o[8];
        read_x(s0 + e, x);
        if (valid <= 0) continue;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = ua.out_scale * x[q];
        const int64_t idx = wrow * wcols + wcol;
        if (!MC_GUARD(2, idx + valid <= static_cast<int64_t>(ua.n) * ua.m)) continue;
        if (vec && valid == 8) {
          u32x4* p = reinterpret_cast<u32x4*>(Wb + idx * kEsz);
          if constexpr (UPD == 3) {
            p[0] = u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                         pack_bf16x2(o[6], o[7])};
          } else if constexpr (UPD == 4) {
            p[0] = __builtin_bit_cast(u32x4, f32x4{o[0], o[1], o[2], o[3]});
            p[1] = __builtin_bit_cast(u32x4, f32x4{o[4], o[5], o[6], o[7]});
          } else if constexpr (UPD == 1) {
            u32x4 w = wbuf[e][0];
            w.x = pack_bf16x2(update_op(bf16_lo(w.x), o[0], ua.lr, ua.wd), update_op(bf16_hi(w.x), o[1], ua.lr, ua.wd));
            w.y = pack_bf16x2(update_op(bf16_lo(w.y), o[2], ua.lr, ua.wd), update_op(bf16_hi(w.y), o[3], ua.lr, ua.wd));
            w.z = pack_bf16x2(update_op(bf16_lo(w.z), o[4], ua.lr, ua.wd), update_op(bf16_hi(w.z), o[5], ua.lr, ua.wd));
            w.w = pack_bf16x2(update_op(bf16_lo(w.w), o[6], ua.lr, ua.wd), update_op(bf16_hi(w.w), o[7], ua.lr, ua.wd));
            p[0] = w;
          } else {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              f32x4 v = __builtin_bit_cast(f32x4, wbuf[e][w]);
              v.x = update_op(v.x, o[4 * w + 0], ua.lr, ua.wd);
              v.y = update_op(v.y, o[4 * w + 1], ua.lr, ua.wd);
              v.z = update_op(v.z, o[4 * w + 2], ua.lr, ua.wd);
              v.w = update_op(v.w, o[4 * w + 3], ua.lr, ua.wd);
              p[w] = __builtin_bit_cast(u32x4, v);
            }
          }
        } else {
          for (int q = 0; q < valid; ++q) {
            if constexpr (UPD == 3) {
              reinterpret_cast<uint16_t*>(Wb)[idx + q] = f32_to_bf16(o[q]);
            } else if constexpr (UPD == 4) {
              reinterpret_cast<float*>(Wb)[idx + q] = o[q];
            } else if constexpr (UPD == 1) {
              uint16_t* pw = reinterpret_cast<uint16_t*>(Wb) + idx + q;
              *pw = f32_to_bf16(update_op(bf16_to_f32(*pw), o[q], ua.lr, ua.wd));
            } else {
              float* pw = reinterpret_cast<float*>(Wb) + idx + q;
              *pw = update_op(*pw, o[q], ua.lr, ua.wd);
            }
          }
        }
      }
    }
    return;
  }
  // direct store: 4 rows of 256 bytes per instruction
  auto store_rows = [&](uint16_t* D) {
#pragma unroll 4
    for (int s = 16 * wh; s < 16 * wh + 16; ++s) {
      const int row = 4 * s + (lane >> 4), u = lane & 15;
      const u32x4 v = *(const lds_u32x4_t*)(uintptr_t)st_addr(row, u);
      const int64_t o = kBlockedOut ? blk_off(i0w + row, j0w + 8 * u, nkb) : x_off(i0w + row, j0w + 8 * u, n_pad);
      if (MC_GUARD(3, o + 8 <= (kBlockedOut ? nn : nm))) *reinterpret_cast<u32x4*>(D + o) = v;
    }
  };
  if constexpr (MODE != 2) {
    store_rows(O);
    if (ti != tj) store_transposed(eb, O, j0w, i0w, nkb, lane, 16 * wh);
  }
}

}  // namespace

MC_DEBUG_UNIT(ns_gemm)

hipError_t launch_ns_gemm(int mode, const NsGeometry& g, const uint16_t* in0, const uint16_t* in1,
                          const uint8_t* xl, uint16_t* out, uint8_t* xl_out, float* dg, float alpha, float beta,
                          float a, const float* inv, const NsUpdate* upd, hipStream_t stream) {
  const int n_pad = static_cast<int>(g.n_pad), m_pad = static_cast<int>(g.m_pad);
  const int tiles_m = n_pad / kBM;
  const int tiles_n = (mode == 2) ? m_pad / kBN : n_pad / kBN;
  // modes 0/1: upper triangle only (symmetric results)
  const int tiles_per_mat = (mode == 2) ? tiles_m * tiles_n : tiles_m * (tiles_m + 1) / 2;
  const int64_t blocks = static_cast<int64_t>(tiles_per_mat) * g.batch;
  dim3 grid(static_cast<unsigned>(blocks));
  UpdArgs ua{};
  if (upd != nullptr) {
    ua.W = upd->W;
    ua.w_stride = upd->w_stride;
    ua.n = static_cast<int>(g.n);
    ua.m = static_cast<int>(g.m);
    ua.out_scale = upd->out_scale;
    ua.lr = upd->lr;
    ua.wd = upd->wd;
  }
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, in0, in1, xl, out, xl_out, dg, n_pad, m_pad,
                       tiles_n, tiles_per_mat, alpha, beta, a, inv, ua);
  };
  const bool sc = inv != nullptr, tr = g.transposed;
  // the last step's epilogue: one instance per scaling and W orientation
  auto go_upd = [&](auto kind) {
    constexpr int U = decltype(kind)::value;
    if (sc) tr ? go(ns_gemm_kernel<2, U, true, true>) : go(ns_gemm_kernel<2, U, true, false>);
    else tr ? go(ns_gemm_kernel<2, U, false, true>) : go(ns_gemm_kernel<2, U, false, false>);
  };
  if (mode == 0) sc ? go(ns_gemm_kernel<0, 0, true, false>) : go(ns_gemm_kernel<0, 0, false, false>);
  else if (mode == 1) go(ns_gemm_kernel<1, 0, false, false>);
  else if (upd == nullptr) sc ? go(ns_gemm_kernel<2, 0, true, false>) : go(ns_gemm_kernel<2, 0, false, false>);
  else if (upd->output && upd->w_bf16) go_upd(std::integral_constant<int, 3>{});
  else if (upd->output) go_upd(std::integral_constant<int, 4>{});
  else if (upd->w_bf16) go_upd(std::integral_constant<int, 1>{});
  else go_upd(std::integral_constant<int, 2>{});
  return hipGetLastError();
}

}  // namespace mc
