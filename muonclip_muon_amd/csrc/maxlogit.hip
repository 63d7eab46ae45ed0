// Per-head max logit, S_max^h = (1/sqrt(d)) max_{b,i,j} Q[b,h,i] . K[b,h,j],
// with the logit matrix never written anywhere ("Kimi K2 内部机制", MuonClip
// section, core maths: max over the batch and over all token pairs).
//
// bf16 path (d_c in {64, 128, 192} and d_r in {0, 64}, d <= 192, Sk >= 64):
//   A 256-thread workgroup (4 wave64s, one per SIMD) owns 512 query rows of
//   one (b, h); each wave keeps its 128 rows of Q as MFMA fragments in
//   registers for the whole kernel, so every key fragment read from LDS feeds
//   4 MFMAs.  Every key row of (b, h) streams through 4 LDS stages of 64 keys
//   x d, filled by LDS DMA (global_load_lds) three blocks ahead, one barrier
//   per block; Kc and Kr rows land in two regions of the stage, so each DMA
//   instruction reads whole rows of one source.  A key block is two phases of
//   32 keys; per phase a wave issues 4 x (d/16) v_mfma_f32_32x32x16_bf16 into
//   one of two accumulator sets while the 128 x 32 logits of the other set
//   (the previous phase) are folded into a 16-register running max between
//   the MFMAs.  The key row is assembled in LDS from the head's own part
//   Kc[b,h,j] and the shared rotary part Kr[b,j] (MLA).  Consecutive
//   workgroups of one (b, h) are kept on one XCD so the key stream is read
//   from that XCD's L2.
// Any other shape (float32, other head dims, Sk < 64) goes to the float32
// LDS-tiled kernel of maxlogit_generic.hip, which keeps NaN semantics.
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

// ------------------------------------------------------------------ bf16 MFMA
constexpr int kMfmaThreads = 256;
constexpr int kRowsPerWave = 128;
constexpr int kRowsPerBlock = kRowsPerWave * (kMfmaThreads / 64);  // 512
constexpr int kKeys = 64;                                          // key rows per LDS stage
constexpr int kKeyStages = 4;                                      // prefetch distance 3

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One global_load_lds_dwordx4: 16 bytes from g_uniform + lane_off to LDS
// address m0 + 16 * lane.  Inline asm so the compiler does not wait for the
// copy before unrelated LDS reads; the copy is awaited with an explicit vmcnt
// wait before the barrier that publishes the stage.  The lane offsets stay
// constant for the whole kernel (the moving part is the uniform base), so no
// register an in-flight copy reads is ever overwritten.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const char* g_uniform, uint32_t lane_off, uint32_t lds_addr) {
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

// Position of 16-byte unit u in key row r of a row of U units.  A fragment
// read (ds_read_b128) serves 16 lanes per cycle, which read one unit of 16
// consecutive rows, so those 16 reads must fall in 16 different 16-byte bank
// groups of the 256-byte bank row: 256-byte rows (U = 16) take u ^ (r & 15);
// rows of 128 or 384 bytes (U = 8, 24), where consecutive rows alternate
// between the two halves of a bank row, take u ^ ((r / 2) & 7), which stays
// inside u's aligned group of 8 units.
template <int U>
__device__ __forceinline__ int kswz(int u, int r) {
  static_assert(U == 1 || U == 16 || U % 16 == 8, "rows of 256 bytes or an odd multiple of 128 bytes");
  if constexpr (U == 1) return u;  // no such part (the loops over it are empty)
  else return U == 16 ? (u ^ (r & 15)) : (u ^ ((r >> 1) & 7));
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Key stage: the 64 key rows' own parts (Kc, DC elements each) in one region
// and their shared rotary parts (Kr, DR each) in another, each row-major; a
// 16-byte unit u of row r sits at position kswz(u, r) of its row (above), so
// the 16 lanes of a fragment read that one cycle serves hit 16 different
// bank groups (SQ_LDS_BANK_CONFLICT 0; with u ^ (r & 7) rows r and r + 8
// shared one and the counter read 4 cycles per LDS instruction, yet the
// kernel was only 0.4 % slower: its LDS reads are not what bounds it).  Every DMA
// instruction then reads whole rows of one source: 1 KB = 1024 / (2 DC) rows
// of Kc, or 1024 / (2 DR) rows of Kr.
template <int DC, int DR>
__global__ __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void maxlogit_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                          const uint16_t* __restrict__ Kr, int H, int Sq, int Sk, int blocks_per_bh,
                          float* __restrict__ smax, float scale) {
  constexpr int D = DC + DR;
  constexpr int kUc = DC / 8, kUr = DR / 8;        // 16-byte units per row and part
  constexpr int kUrNz = kUr > 0 ? kUr : 1;          // divisor for the Kr loop, which is empty when DR = 0
  constexpr int kSteps = D / 16;                   // MFMA k-steps
  constexpr int kKcBytes = kKeys * DC * 2, kKrBytes = kKeys * DR * 2;
  constexpr int kStageBytes = kKcBytes + kKrBytes;
  constexpr int kLoadsC = kKcBytes / 1024 / 4, kLoadsR = kKrBytes / 1024 / 4;  // per wave
  constexpr int kLoads = kLoadsC + kLoadsR;
  static_assert(DC % 64 == 0 && DR % 64 == 0, "parts of 64-element multiples");
  __shared__ __attribute__((aligned(1024))) char smem[kKeyStages * kStageBytes];
  __shared__ float red[kMfmaThreads / 64];
  typedef __attribute__((address_space(3))) char lds_char_t;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));

  const uint32_t bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = bid / blocks_per_bh;
  const int ib = bid % blocks_per_bh;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int frag_row = lane & 31, frag_half = lane >> 5;

  const uint16_t* Qbh = Q + (static_cast<int64_t>(b) * H + h) * Sq * D;
  const char* Kcbh = reinterpret_cast<const char*>(Kc + (static_cast<int64_t>(b) * H + h) * Sk * DC);
  const char* Krb = reinterpret_cast<const char*>(Kr ? Kr + static_cast<int64_t>(b) * Sk * DR : Kc);

  // ---- key loads.  DMA instruction l of this wave fills 1 KB at region
  // offset 1024 (wave + 4 l); its lane slot p = 64 (wave + 4 l) + lane holds
  // row r = p / units, unit kswz(p % units, r).  Lane offsets are relative
  // to key row j0 of the block, which moves with the uniform base.
  uint32_t off_c[kLoadsC > 0 ? kLoadsC : 1], off_r[kLoadsR > 0 ? kLoadsR : 1];
#pragma unroll
  for (int l = 0; l < kLoadsC; ++l) {
    const int p = 64 * (wave + 4 * l) + lane;
    const int r = p / kUc, u = kswz<kUc>(p % kUc, r);
    off_c[l] = static_cast<uint32_t>((r * DC + 8 * u) * 2);
  }
#pragma unroll
  for (int l = 0; l < kLoadsR; ++l) {
    const int p = 64 * (wave + 4 * l) + lane;
    const int r = p / kUrNz, u = kswz<kUrNz>(p % kUrNz, r);
    off_r[l] = static_cast<uint32_t>((r * DR + 8 * u) * 2);
  }
  const int NJ = (Sk + kKeys - 1) / kKeys;
  // DMA instruction l (of kLoads) of block jb: Kc parts first, then Kr
  auto issue_part = [&](int jb, int l) {
    const int64_t j0 = min(min(jb, NJ - 1) * kKeys, Sk - kKeys);
    const uint32_t st = lds + (jb % kKeyStages) * kStageBytes;
    if (!MC_GUARD(1, j0 >= 0 && j0 + kKeys <= Sk)) return;
    if (l < kLoadsC) load_lds16(Kcbh + j0 * DC * 2, off_c[l], st + 1024 * (wave + 4 * l));
    else load_lds16(Krb + j0 * DR * 2, off_r[l - kLoadsC], st + kKcBytes + 1024 * (wave + 4 * (l - kLoadsC)));
  };
  auto issue = [&](int jb) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) issue_part(jb, l);
  };
  // the first kKeyStages - 1 key blocks, issued before Q's loads
  for (int s = 0; s < kKeyStages - 1; ++s) issue(s);

  // ---- this wave's 128 query rows as MFMA "A" fragments (row = lane % 32).
  // Tails need no masking: a query row past Sq repeats row Sq - 1, and the
  // last key block is the last 64 keys (it may overlap the previous one), so
  // every logit computed is one of the real ones and the maximum is exact.
  const int row_base = ib * kRowsPerBlock + wave * kRowsPerWave;
  bf16x8 qf[4][kSteps];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = min(row_base + t * 32 + frag_row, Sq - 1);
    const bool ok = MC_GUARD(0, i >= 0 && i < Sq);
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qf[t][s] = ok ? as_bf16x8(*reinterpret_cast<const u32x4*>(Qbh + static_cast<int64_t>(i) * D + 16 * s + 8 * frag_half))
                    : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  // Q is in registers before the loop: otherwise the compiler, which cannot
  // tell the key copies from these loads, waits on the copies in flight
  // before the first use of each Q register inside the loop.  The empty asm
  // statements consume every Q register (forcing the loads to complete,
  // together with the first key copies issued before them, so the two
  // latencies overlap) and, being volatile, stay ahead of the later copies.
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < kSteps; ++s) asm volatile("" : : "v"(qf[t][s]));


  // ---- main loop.  A key block is two phases of 32 keys (u = 0, 1); a
  // phase is kSteps k-steps of 4 MFMAs (one per 32-row query tile t) into
  // acc[t][u].  The two halves double-buffer the logits: while phase u runs
  // its MFMAs, the 64 logits per lane of the other half (the phase before)
  // are folded into the running max a few rows per step, so the VALU work
  // issues between MFMAs instead of after them.  This file is built with MFMA
  // results in VGPRs and without NaN semantics for float operations, so a
  // fold is one v_max3_f32 per two logits, read straight from the MFMA result
  // registers.  Key fragments are read two
  // steps ahead through 4 buffers (the flat step count per block is a
  // multiple of 4, so buffer indices repeat every block); the reads of the
  // next block's first two steps go out under this block's last two steps,
  // after the barrier that publishes its stage.
  constexpr int kBlockSteps = 2 * kSteps;
  constexpr int kBarrierStep = kBlockSteps - 2;
  constexpr int kEvery = (kBlockSteps + kLoads - 1) / kLoads;  // steps between refill DMAs
  // refill DMAs of this block issued before its barrier
  constexpr int kIssuedBefore = ((kBarrierStep - 1) / kEvery + 1) < kLoads ? ((kBarrierStep - 1) / kEvery + 1) : kLoads;
  static_assert(kBlockSteps % 4 == 0, "fragment buffers repeat every block");
  static_assert(kSteps >= 3, "the fold is spread over steps 1 .. kSteps - 1");

  // fragment of flat step f (phase f / kSteps, k-step f % kSteps) of a stage
  auto read_kf = [&](uint32_t stage, int f) -> bf16x8 {
    const int u = f / kSteps, s = f % kSteps;
    const int unit = 2 * s + frag_half;  // of the full row of D
    const int row = u * 32 + frag_row;
    // 2 s < DC / 8 decides the part at compile time (both parts hold an even
    // number of units)
    const uint32_t a = (2 * s < kUc) ? stage + row * (2 * DC) + 16 * kswz<kUc>(unit, row)
                                     : stage + kKcBytes + row * (2 * DR) + 16 * kswz<kUrNz>(unit - kUc, row);
    return as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)a);
  };

  f32x16 run, acc[4][2];
#pragma unroll
  for (int r = 0; r < 16; ++r) run[r] = -INFINITY;
  // the half folded during the very first phase holds no logits yet
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t][1] = run;

  // block 0's loads are older than the 2 newer stages in flight (the wait
  // for Q above has already covered them)
  wait_vmem<(kKeyStages - 2) * kLoads>();
  __syncthreads();
  bf16x8 kf[4];
  kf[0] = read_kf(lds, 0);
  kf[1] = read_kf(lds, 1);

  for (int jb = 0; jb < NJ; ++jb) {
    const uint32_t cur = lds + (jb % kKeyStages) * kStageBytes;
    const uint32_t nxt = lds + ((jb + 1) % kKeyStages) * kStageBytes;
#pragma unroll
    for (int f = 0; f < kBlockSteps; ++f) {
      const int u = f / kSteps, s = f % kSteps;
      if (f == kBarrierStep) {
        // block jb + 1 has landed (only block jb + 2 and this block's
        // refills are newer); every read of this block's stage has been
        // issued, so after the barrier its stage may be refilled as well
        wait_vmem<kLoads + kIssuedBefore>();
        __syncthreads();
      }
      const int g = f + 2;
      kf[g % 4] = (g < kBlockSteps) ? read_kf(cur, g) : read_kf(nxt, g - kBlockSteps);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], kf[f % 4], s == 0 ? f32x16{} : acc[t][u],
                                                            0, 0, 0);
      // fold rows r of the other half whose turn is this step: rows spread
      // evenly over steps 1 .. kSteps - 1 (step 0 leaves the last MFMAs of
      // the other half time to finish)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (s == 1 + r * (kSteps - 1) / 16) {
          const int o = 1 - u;
          run[r] = fmaxf(fmaxf(run[r], acc[0][o][r]), acc[1][o][r]);
          run[r] = fmaxf(fmaxf(run[r], acc[2][o][r]), acc[3][o][r]);
        }
      }
      // one DMA instruction of the refill (block jb + 3) every kEvery steps
      if (f % kEvery == 0 && f / kEvery < kLoads) issue_part(jb + kKeyStages - 1, f / kEvery);
    }
  }
  // the last phase's half
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    run[r] = fmaxf(fmaxf(run[r], acc[0][1][r]), acc[1][1][r]);
    run[r] = fmaxf(fmaxf(run[r], acc[2][1][r]), acc[3][1][r]);
  }
  wait_vmem<0>();  // the redundant prefetches past the last block

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
    if (w != -INFINITY && MC_GUARD(2, h >= 0 && h < H)) atomic_max_float(&smax[h], w * scale);
  }
}

template <int DC, int DR>
hipError_t launch_mfma(const void* Q, const void* Kc, const void* Kr, int64_t B, int64_t H, int64_t Sq,
                       int64_t Sk, float* smax, float scale, hipStream_t stream) {
  const int64_t blocks_per_bh = (Sq + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = blocks_per_bh * B * H;
  hipLaunchKernelGGL((maxlogit_mfma_kernel<DC, DR>), dim3(static_cast<unsigned>(blocks)), dim3(kMfmaThreads),
                     0, stream, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(Kc),
                     static_cast<const uint16_t*>(Kr), static_cast<int>(H), static_cast<int>(Sq),
                     static_cast<int>(Sk), static_cast<int>(blocks_per_bh), smax, scale);
  return hipGetLastError();
}

}  // namespace

MC_DEBUG_UNIT(maxlogit)

hipError_t launch_maxlogit(const void* Q, const void* Kc, const void* Kr, bool bf16, int64_t B,
                           int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                           hipStream_t stream) {
  const int64_t d = d_c + d_r;
  const float scale = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
  const bool aligned16 = (reinterpret_cast<uintptr_t>(Q) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(Kc) % 16 == 0) &&
                         (Kr == nullptr || reinterpret_cast<uintptr_t>(Kr) % 16 == 0);
  // MFMA kernel shapes: parts of 64-element multiples, d <= 192, at least one
  // full key block (the last block is the last 64 keys)
  const bool mfma_ok = bf16 && aligned16 && Sk >= kKeys && Sq <= INT32_MAX && Sk <= INT32_MAX &&
                       B * H * ((Sq + kRowsPerBlock - 1) / kRowsPerBlock) <= INT32_MAX &&
                       (Kr != nullptr || d_r == 0);
  if (mfma_ok) {
    if (d_c == 64 && d_r == 0) return launch_mfma<64, 0>(Q, Kc, Kr, B, H, Sq, Sk, smax, scale, stream);
    if (d_c == 128 && d_r == 0) return launch_mfma<128, 0>(Q, Kc, Kr, B, H, Sq, Sk, smax, scale, stream);
    if (d_c == 192 && d_r == 0) return launch_mfma<192, 0>(Q, Kc, Kr, B, H, Sq, Sk, smax, scale, stream);
    if (d_c == 64 && d_r == 64) return launch_mfma<64, 64>(Q, Kc, Kr, B, H, Sq, Sk, smax, scale, stream);
    if (d_c == 128 && d_r == 64) return launch_mfma<128, 64>(Q, Kc, Kr, B, H, Sq, Sk, smax, scale, stream);
  }
  return launch_maxlogit_generic(Q, Kc, Kr, bf16, B, H, Sq, Sk, d_c, d_r, smax, scale, stream);
}

}  // namespace mc
