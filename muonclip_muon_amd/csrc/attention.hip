// Attention forward with the per-head max logit as a by-product:
//   O[b,h,i] = sum_j softmax_j(Q[b,h,i] . K[b,h,j] / sqrt(d)) V[b,h,j],
//   S_max^h  = max_{b,i,j} Q[b,h,i] . K[b,h,j] / sqrt(d)   (visible j only),
// with K[b,h,j] = [Kc[b,h,j] || Kr[b,j]] (MLA: the rotary key is shared by all
// heads) or Kc alone (MHA), and an optional causal mask (query i sees key j
// when j <= i + Sk - Sq).  "Kimi K2 内部机制", MuonClip section: S_max is
// already computed in the forward; the paper notes (section 3.2) read the
// per-head max logit from the attention forward.  The logits never leave
// registers; the running row maximum of the softmax is the max logit.
//
// bf16, (d_c, d_r, d_v) in {(128, 64, 128), (64, 0, 64)}, Sk >= 64.
// A 256-thread workgroup (4 wave64s) owns 256 query rows of one (b, h); each
// wave keeps its 64 rows of Q as MFMA fragments in registers.  Keys and
// values stream through 4 LDS stages of 64 keys (K rows and V rows, filled by
// LDS DMA three blocks ahead, one barrier per block).  A block is two phases of
// 32 keys; per phase and wave:
//   S = K Q^T     2 x (d/16) v_mfma_f32_32x32x16_bf16 (keys as the MFMA rows,
//                 so each lane holds 16 keys of one query row);
//   softmax       row max over the lane's 16 keys and the other half-wave's
//                 16 (one lane swap), p = 2^(s log2(e)/sqrt(d) - m) in float32,
//                 rounded to bf16 for the second product; the row sum stays a
//                 per-lane partial until the end;
//   O += V^T P    (d_v/32) x 2 x 2 MFMAs (d as the MFMA rows), P straight from
//                 the registers of S: the MFMA k order is permuted to the
//                 order in which S holds the keys, and the V fragments are
//                 read in that order with ds_read_b64_tr_b16.
// The reference point m of the exponentials follows the row maximum lazily:
// it moves (and O and the row sum are rescaled by 2^(m_old - m_new)) only
// when a block's maximum exceeds it by more than 32 (so p <= 2^32, and the row
// sums stay far from the float32 and bf16 range limits), which keeps the
// result exact up to rounding and makes the rescale rare.  The true row
// maximum is tracked separately for S_max.
//
// Tails: a query row past Sq repeats row Sq - 1 and is not stored; the last
// key block is the last 64 keys (in bounds) with the keys of the previous
// block masked out.  Workgroups whose rows cannot see a key block under the
// causal mask stop before it.

#include <math.h>

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / 64);  // 256
constexpr int kKeys = 64;                                     // keys per LDS stage
constexpr int kStages = 4;                                    // prefetch distance 3
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 32.0f;  // log2 units the reference may lag the row max

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One global_load_lds_dwordx4: 16 bytes from g_uniform + lane_off to LDS
// address m0 + 16 * lane; completion is awaited with an explicit vmcnt wait
// before the barrier that publishes the stage.
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

template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// x of this lane and of lane l ^ 32 (the other half-wave), with
// v_permlane32_swap: the swap of the upper half of its first operand with the
// lower half of its second leaves, with both operands x, the two values in
// the two results.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// LDS layout of a stage: K rows (the Kc part, then the Kr part, each its own
// row-major region; 16-byte unit u of row r at position kswz(u, r, units)),
// then V rows (row-major, unit u of row r at u ^ vswz(r)).  A key fragment
// read (ds_read_b128) serves 16 lanes per cycle, one unit of 16 consecutive
// rows, so kswz puts those in 16 different 16-byte bank groups of a 256-byte
// bank row: u ^ (r & 15) for 256-byte rows, u ^ ((r / 2) & 7) for 128-byte
// rows (consecutive rows alternate between the halves of a bank row).  vswz
// spreads the 4 rows a transposed read touches (rows r .. r + 3, r % 4 == 0)
// over different banks.
__device__ __forceinline__ int kswz(int u, int r, int units) {
  return units == 16 ? (u ^ (r & 15)) : units == 8 ? (u ^ ((r >> 1) & 7)) : u;
}
template <int DV>
__device__ __forceinline__ int vswz(int r) {
  return DV == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int DC, int DR, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                          const uint16_t* __restrict__ Kr, const uint16_t* __restrict__ V, int H, int Sq,
                          int Sk, int blocks_per_bh, int causal, float c_log2, float inv_sqrt_d,
                          uint16_t* __restrict__ O, float* __restrict__ lse, float* __restrict__ smax) {
  constexpr int D = DC + DR;
  constexpr int kUc = DC / 8, kUr = DR / 8, kUv = DV / 8;  // 16-byte units per row
  constexpr int kSteps = D / 16;                           // k16 steps of S = K Q^T
  constexpr int kDt = DV / 32;                             // 32-row MFMA tiles of O
  constexpr int kKcBytes = kKeys * DC * 2, kKrBytes = kKeys * DR * 2, kVBytes = kKeys * DV * 2;
  constexpr int kStageBytes = kKcBytes + kKrBytes + kVBytes;
  constexpr int kLoadsC = kKcBytes / 4096, kLoadsR = kKrBytes / 4096, kLoadsV = kVBytes / 4096;  // per wave
  constexpr int kLoads = kLoadsC + kLoadsR + kLoadsV;
  static_assert(DC % 64 == 0 && DR % 64 == 0 && (DV == 64 || DV == 128), "supported head dims");
  static_assert(kLoads <= kSteps, "one block's copies fit one phase, one every other slot");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));

  const uint32_t bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = bid / blocks_per_bh;
  const int ib = bid % blocks_per_bh;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int frag_row = lane & 31, frag_half = lane >> 5;

  const int64_t bh64 = static_cast<int64_t>(b) * H + h;
  const uint16_t* Qbh = Q + bh64 * Sq * D;
  const char* Kcbh = reinterpret_cast<const char*>(Kc + bh64 * Sk * DC);
  const char* Krb = reinterpret_cast<const char*>(DR > 0 ? Kr + static_cast<int64_t>(b) * Sk * DR : Kc);
  const char* Vbh = reinterpret_cast<const char*>(V + bh64 * Sk * DV);
  const int off = Sk - Sq;  // causal: query i sees keys j <= i + off

  // ---- this wave's 64 query rows as MFMA "B" fragments (column = lane % 32)
  const int row_base = ib * kRowsPerBlock + wave * kRowsPerWave;
  bf16x8 qf[2][kSteps];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = min(row_base + t * 32 + frag_row, Sq - 1);
    const bool ok = MC_GUARD(0, i >= 0 && i < Sq);
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qf[t][s] = ok ? as_bf16x8(*reinterpret_cast<const u32x4*>(Qbh + static_cast<int64_t>(i) * D + 16 * s + 8 * frag_half))
                    : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  // Q in registers before any copy starts (the copies' asm is opaque to the
  // compiler, which would otherwise wait on them before each use of Q), and
  // in AGPRs, which MFMA reads directly: the VGPRs hold the softmax.
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < kSteps; ++s) asm volatile("" : "+a"(qf[t][s]));

  // ---- key / value loads: DMA instruction l of this wave fills 1 KB at
  // region offset 1024 (wave + 4 l); lane slot p = 64 (wave + 4 l) + lane holds
  // row p / units, unit (p % units) ^ swizzle(row).  Every region has rows of
  // 128 or 256 bytes, so 4 KB further (l + 1) is a whole number of rows that
  // leaves the row's swizzle unchanged: one lane offset per region, and the
  // 4 KB steps go into the uniform base.
  auto lane_off = [&](int units, int row_elems, int kind) -> uint32_t {
    const int p = 64 * wave + lane;
    const int r = p / units;
    const int u = kind == 2 ? (p % units) ^ vswz<DV>(r) : kswz(p % units, r, units);
    return static_cast<uint32_t>((r * row_elems + 8 * u) * 2);
  };
  const uint32_t lo_c = lane_off(kUc, DC, 0), lo_r = lane_off(kUr > 0 ? kUr : 1, DR, 1), lo_v = lane_off(kUv, DV, 2);
  const int NJ = (Sk + kKeys - 1) / kKeys;
  // key blocks this workgroup needs: all, or up to the last key its last row sees
  int nj = NJ;
  if (causal) {
    const int last_row = min(ib * kRowsPerBlock + kRowsPerBlock - 1, Sq - 1);
    nj = min(NJ, (min(Sk - 1, last_row + off)) / kKeys + 1);
  }
  auto block_start = [&](int jb) { return min(min(jb, NJ - 1) * kKeys, Sk - kKeys); };
  // DMA instruction l (of kLoads: the Kc parts, the Kr parts, the V parts) of block jb
  auto issue_part = [&](int jb, int l) {
    const int64_t j0 = block_start(jb);
    const uint32_t st = lds + (jb % kStages) * kStageBytes;
    if (!MC_GUARD(1, j0 >= 0 && j0 + kKeys <= Sk)) return;
    if (l < kLoadsC) {
      load_lds16(Kcbh + j0 * DC * 2 + 4096 * l, lo_c, st + 1024 * (wave + 4 * l));
    } else if (l < kLoadsC + kLoadsR) {
      const int m = l - kLoadsC;
      load_lds16(Krb + j0 * DR * 2 + 4096 * m, lo_r, st + kKcBytes + 1024 * (wave + 4 * m));
    } else {
      const int m = l - kLoadsC - kLoadsR;
      load_lds16(Vbh + j0 * DV * 2 + 4096 * m, lo_v, st + kKcBytes + kKrBytes + 1024 * (wave + 4 * m));
    }
  };
  auto issue = [&](int jb) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) issue_part(jb, l);
  };

  // running state per query tile t (this lane's row i = row_base + 32 t + lane % 32)
  f32x16 oacc[kDt][2];
#pragma unroll
  for (int a = 0; a < kDt; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) oacc[a][t] = f32x16{};
  float m_ref[2] = {-INFINITY, -INFINITY};   // reference of the exponentials (log2 units)
  float m_true[2] = {-INFINITY, -INFINITY};  // true row max of the raw logits
  float l_sum[2] = {0.f, 0.f};               // this lane's part of the row sum
  int row_i[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) row_i[t] = min(row_base + t * 32 + frag_row, Sq - 1);

  // Per-lane LDS read offsets with everything that is a compile-time constant
  // left out: K fragments (row lane % 32, unit 2 s + half) repeat their
  // swizzle every 4 k-steps: in a 256-byte row k-steps 4..7 are units 8..15,
  // which kswz puts at the offset of units 0..7 with bit 7 flipped, so 4
  // offsets per K part cover every step (XOR 128 for steps 4..7, + 32 rows
  // per phase); V transposed reads depend on the column tile only (the
  // phase, k16 step and upper rows are whole multiples of 4 rows).
  uint32_t kc_off[4], kr_off[4], v_off[kDt];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const int unit = 2 * s4 + frag_half;
    kc_off[s4] = frag_row * (2 * DC) + 16 * kswz(unit, frag_row, kUc);
    kr_off[s4] = kKcBytes + frag_row * (2 * DR) + 16 * kswz(unit, frag_row, kUr);
  }
  {
    const int g = lane >> 4, il = lane & 15;
    const int r = 4 * (g >> 1) + (il >> 2);
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const int col = 32 * dt + 16 * (g & 1) + 4 * (il & 3);
      v_off[dt] = kKcBytes + kKrBytes + r * (2 * DV) + (((col >> 3) ^ vswz<DV>(r)) << 4) + (col & 7) * 2;
    }
  }

  f32x16 sA[2], sB[2];
  bf16x8 pf[2][2];
  float alpha[2];
  // ---- the three parts of a phase
  // S = K Q^T for keys 32 u .. + 31 of the stage at st
  auto qk = [&](uint32_t st, int u, f32x16 (&S)[2]) {
    S[0] = f32x16{};
    S[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      // 2 s < DC / 8 decides the part at compile time
      const int sp = (2 * s < kUc) ? s : s - kUc / 2;  // k-step within the part
      const uint32_t a = (2 * s < kUc) ? st + (kc_off[sp & 3] ^ (128 * (sp >> 2))) + u * 32 * (2 * DC)
                                       : st + (kr_off[sp & 3] ^ (128 * (sp >> 2))) + u * 32 * (2 * DR);
      const bf16x8 kf = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)a);
#pragma unroll
      for (int t = 0; t < 2; ++t) S[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t][s], S[t], 0, 0, 0);
    }
  };
  // Softmax of one phase as a list of small work items, so it can be spread
  // between the MFMAs of the next phase's S (see qk_softmax).  Register r of
  // S[t] holds key j0 + 32 u + 8 (r / 4) + 4 half + r % 4 of row row_i[t].
  // Items: [mask t0 lo, t0 hi, t1 lo, t1 hi] (masked phases only), max t0,
  // max t1, reference t0, reference t1, then 8 exponential pairs per t.  Each
  // pair is packed to bf16 at once and added to a partial row sum.
  float mb[2], psum[2], mr[2];
  auto softmax_item = [&](f32x16 (&S)[2], bool mask, int j0, int j_lo, int u, int item) {
    if (mask) {
      if (item < 4) {
        const int t = item >> 1, r0 = 8 * (item & 1);
#pragma unroll
        for (int r = r0; r < r0 + 8; ++r) {
          const int j = j0 + 32 * u + 8 * (r >> 2) + 4 * frag_half + (r & 3);
          S[t][r] = (j < j_lo || (causal && j > row_i[t] + off)) ? -INFINITY : S[t][r];
        }
        return;
      }
      item -= 4;
    }
    if (item < 2) {  // row max over this lane's 16 keys
      const int t = item;
      mb[t] = fmaxf(fmaxf(fmaxf(fmaxf(S[t][0], S[t][1]), fmaxf(S[t][2], S[t][3])),
                          fmaxf(fmaxf(S[t][4], S[t][5]), fmaxf(S[t][6], S[t][7]))),
                    fmaxf(fmaxf(fmaxf(S[t][8], S[t][9]), fmaxf(S[t][10], S[t][11])),
                          fmaxf(fmaxf(S[t][12], S[t][13]), fmaxf(S[t][14], S[t][15]))));
      return;
    }
    if (item < 4) {  // the other half-wave's keys; move the reference lazily
      const int t = item - 2;
      float x, y;
      halves(mb[t], x, y);
      const float m = fmaxf(x, y);
      m_true[t] = fmaxf(m_true[t], m);
      const float m2 = m * c_log2;
      const float m_new = (m2 > m_ref[t] + kRescaleSlack) ? m2 : m_ref[t];
      alpha[t] = (m_new == m_ref[t]) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[t] - m_new);
      m_ref[t] = m_new;
      // a row that has seen no visible key yet keeps p = 0 (no inf - inf)
      mr[t] = m_new == -INFINITY ? 0.f : m_new;
      psum[t] = 0.f;
      return;
    }
    item -= 4;  // exponential pair: t = item / 8, registers 2 (item % 8), + 1
    const int t = item >> 3, r = 2 * (item & 7);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(S[t][r], c_log2, -mr[t]));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(S[t][r + 1], c_log2, -mr[t]));
    psum[t] += p0 + p1;
    u32x4 w = __builtin_bit_cast(u32x4, pf[t][r >> 3]);
    w[(r & 7) >> 1] = pack_bf16x2(p0, p1);
    pf[t][r >> 3] = __builtin_bit_cast(bf16x8, w);
  };
  // O = alpha O (rare: a wave-uniform branch) and O += V^T P for keys
  // 32 u .. + 31 of the stage at st.  k16 step t16 covers keys 16 t16 .. + 15
  // of the phase in the order S holds them: half h's slots e = 0..3 are keys
  // 4 h + e, slots 4..7 keys 8 + 4 h + e - 4.  Lane (16-lane group g, i) of a
  // transposed read addresses V row 4 (g / 2) + i / 4 (+ 8 for slots 4..7),
  // columns 32 dt + 16 (g & 1) + 4 (i & 3) .. + 3.
  // V fragment of k16 step t16 and column tile dt of phase u (two transposed reads)
  auto read_vf = [&](uint32_t st, int u, int t16, int dt) -> bf16x8 {
    const uint32_t a = st + v_off[dt] + (32 * u + 16 * t16) * (2 * DV);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)a);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)(a + 8 * (2 * DV)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return as_bf16x8(u32x4{l2.x, l2.y, h2.x, h2.y});
  };
  bf16x8 vpre[kDt];  // the phase's t16 = 0 fragments, read under the QK MFMAs
  auto pv = [&](uint32_t st, int u, const bf16x8 (&pf)[2][2], const float (&alpha)[2]) {
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int a = 0; a < kDt; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[a][t][r] *= alpha[t];
    }
#pragma unroll
    for (int t16 = 0; t16 < 2; ++t16) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const bf16x8 vf = t16 == 0 ? vpre[dt] : read_vf(st, u, 1, dt);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          oacc[dt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t][t16], oacc[dt][t], 0, 0, 0);
      }
    }
  };
  // S of the next phase with the softmax of the current one, interleaved by
  // hand (the scheduler otherwise puts every MFMA first): per k-step, the two
  // MFMAs each followed by the softmax items of that slot, fenced so the
  // order stays; K fragments are read two steps ahead.  Then the row sums.
  // st_v / u: the current phase (its V fragments of k16 step 0 are read in
  // the last slots); dma_block >= 0: that block's copies go out one every
  // other slot.
  auto qk_softmax = [&](uint32_t st, int u_next, f32x16 (&Sn)[2], f32x16 (&Sc)[2], bool mask, int j0, int j_lo,
                        int u, uint32_t st_v, int dma_block) {
    constexpr int kSlots = 2 * kSteps;
    const int n_items = (mask ? 4 : 0) + 4 + 16;
    auto kaddr = [&](int s) -> uint32_t {
      const int sp = (2 * s < kUc) ? s : s - kUc / 2;  // k-step within the part
      return (2 * s < kUc) ? st + (kc_off[sp & 3] ^ (128 * (sp >> 2))) + u_next * 32 * (2 * DC)
                           : st + (kr_off[sp & 3] ^ (128 * (sp >> 2))) + u_next * 32 * (2 * DR);
    };
    bf16x8 kf[3];
    kf[0] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)kaddr(0));
    if (kSteps > 1) kf[1] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)kaddr(1));
    Sn[0] = f32x16{};
    Sn[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s + 2 < kSteps) kf[(s + 2) % 3] = as_bf16x8(*(const lds_u32x4_t*)(uintptr_t)kaddr(s + 2));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        Sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3], qf[t][s], Sn[t], 0, 0, 0);
        const int slot = 2 * s + t;
        // items i with i * kSlots / n_items == slot
#pragma unroll
        for (int i = 0; i < 24; ++i)
          if (i < n_items && (i * kSlots) / n_items == slot) softmax_item(Sc, mask, j0, j_lo, u, i);
        if (dma_block >= 0 && (slot & 1) == 0 && slot / 2 < kLoads) issue_part(dma_block, slot / 2);
        if (slot >= kSlots - kDt) vpre[slot - (kSlots - kDt)] = read_vf(st_v, u, 0, slot - (kSlots - kDt));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) l_sum[t] = fmaf(l_sum[t], alpha[t], psum[t]);  // per lane until the end
  };
  // masks only where some key of the phase is hidden from some row of the wave
  auto needs_mask = [&](int jb, int u) {
    const int j0 = block_start(jb), j_lo = jb * kKeys;
    return (j0 + 32 * u < j_lo) || (causal && j0 + 32 * u + 31 > row_base + off);
  };

  // ---- main loop, software-pipelined by one phase: the S of the next phase
  // is computed while the current phase's softmax runs (independent work for
  // the MFMA and vector units), then the current phase's O += V^T P.  Block
  // jb uses stage jb % 4 (its own K and V) and, in its second phase, the K
  // of stage jb + 1; the barrier between its phases publishes stage jb + 1
  // and frees stage jb - 1 (last read in phase 2 jb - 1), which is refilled
  // with block jb + 3.
  for (int s0 = 0; s0 < kStages - 1; ++s0) issue(s0);
  wait_vmem<(kStages - 2) * kLoads>();  // block 0 landed
  __syncthreads();
  qk(lds, 0, sA);
  for (int jb = 0; jb < nj; ++jb) {
    // O stays in AGPRs across the iteration: without this the compiler keeps
    // a VGPR copy of it for the (rare) rescale and refreshes it every block
#pragma unroll
    for (int a = 0; a < kDt; ++a)
#pragma unroll
      for (int t = 0; t < 2; ++t) asm volatile("" : "+a"(oacc[a][t]));
    const uint32_t st = lds + (jb % kStages) * kStageBytes;
    const uint32_t st1 = lds + ((jb + 1) % kStages) * kStageBytes;
    const int j0 = block_start(jb), j_lo = jb * kKeys;
    // phase 0: S of phase 1 (same stage) with the softmax of phase 0
    if (needs_mask(jb, 0)) qk_softmax(st, 1, sB, sA, true, j0, j_lo, 0, st, -1);
    else qk_softmax(st, 1, sB, sA, false, j0, j_lo, 0, st, -1);
    pv(st, 0, pf, alpha);
    wait_vmem<kLoads>();  // block jb + 1 landed; only block jb + 2 is newer
    __syncthreads();
    // phase 1: S of the next block's phase 0 (past the last block a redundant
    // copy of it) with the softmax of phase 1
    // block jb + 3's copies (into the stage freed by the barrier) go out
    // under this phase's MFMAs
    if (needs_mask(jb, 1)) qk_softmax(st1, 0, sA, sB, true, j0, j_lo, 1, st, jb + kStages - 1);
    else qk_softmax(st1, 0, sA, sB, false, j0, j_lo, 1, st, jb + kStages - 1);
    pv(st, 1, pf, alpha);
  }
  wait_vmem<0>();  // the prefetches past the last block

  // ---- epilogue: O = acc / row sum (both half-waves' parts), LSE, S_max
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float la, lb;
    halves(l_sum[t], la, lb);
    const float l_tot = la + lb;
    const float inv = 1.0f / l_tot;
    const int i = row_base + t * 32 + frag_row;
    if (i < Sq && MC_GUARD(2, i >= 0)) {
      uint16_t* orow = O + (bh64 * Sq + i) * DV;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = 32 * dt + 8 * g4 + 4 * frag_half;
          const u32x2 w = {pack_bf16x2(oacc[dt][t][4 * g4 + 0] * inv, oacc[dt][t][4 * g4 + 1] * inv),
                           pack_bf16x2(oacc[dt][t][4 * g4 + 2] * inv, oacc[dt][t][4 * g4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d) = w;
        }
      if (lse != nullptr && frag_half == 0) lse[bh64 * Sq + i] = (m_ref[t] + log2f(l_tot)) * (1.0f / kLog2e);
    }
  }
  float m = fmaxf(m_true[0], m_true[1]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  // the stages are free: every copy has landed and every wave is past its reads
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) {
    float w = red[0];
    for (int k = 1; k < kThreads / 64; ++k) w = fmaxf(w, red[k]);
    if (w != -INFINITY) atomic_max_float(&smax[h], w * inv_sqrt_d);
  }
}

template <int DC, int DR, int DV>
hipError_t launch(const void* Q, const void* Kc, const void* Kr, const void* V, int64_t B, int64_t H,
                  int64_t Sq, int64_t Sk, bool causal, void* O, float* lse, float* smax, hipStream_t stream) {
  const int64_t blocks_per_bh = (Sq + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = blocks_per_bh * B * H;
  const double d = static_cast<double>(DC + DR);
  const float c_log2 = static_cast<float>(1.4426950408889634 / sqrt(d));
  const float inv_sqrt_d = static_cast<float>(1.0 / sqrt(d));
  hipLaunchKernelGGL((attention_fwd_kernel<DC, DR, DV>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(Kc),
                     static_cast<const uint16_t*>(Kr), static_cast<const uint16_t*>(V), static_cast<int>(H),
                     static_cast<int>(Sq), static_cast<int>(Sk), static_cast<int>(blocks_per_bh), causal ? 1 : 0,
                     c_log2, inv_sqrt_d, static_cast<uint16_t*>(O), lse, smax);
  return hipGetLastError();
}

}  // namespace

MC_DEBUG_UNIT(attention)

bool attention_fwd_supported(int64_t d_c, int64_t d_r, int64_t d_v) {
  return (d_c == 128 && d_r == 64 && d_v == 128) || (d_c == 64 && d_r == 0 && d_v == 64);
}

hipError_t launch_attention_fwd(const void* Q, const void* Kc, const void* Kr, const void* V, int64_t B,
                                int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, int64_t d_v,
                                bool causal, void* O, float* lse, float* smax, hipStream_t stream) {
  if (d_c == 128 && d_r == 64 && d_v == 128)
    return launch<128, 64, 128>(Q, Kc, Kr, V, B, H, Sq, Sk, causal, O, lse, smax, stream);
  if (d_c == 64 && d_r == 0 && d_v == 64)
    return launch<64, 0, 64>(Q, Kc, Kr, V, B, H, Sq, Sk, causal, O, lse, smax, stream);
  return hipErrorInvalidValue;
}

}  // namespace mc
