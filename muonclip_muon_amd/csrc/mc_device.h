// Device-side helpers shared by the kernel translation units of libmuonclip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mc {

// Native clang vector types (HIP's float4/uint4 are structs, which the
// nontemporal and MFMA builtins do not accept).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bfloat16 <-> float32.  bfloat16 is the upper half of a binary32, so the
// widening is a shift.  The narrowing is gfx950's v_cvt_pk_bf16_f32 (two
// values per instruction, round to nearest even, NaNs stay NaN), reached
// through a plain float -> __bf16 conversion; a bit-twiddling version costs a
// branch per value for the NaN case.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> two packed bfloat16 in one dword (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The rounding of the element-wise steps, shared by every kernel that applies
// them.  Each is a chain of separate float32 operations, each rounded once,
// with FP contraction switched off (clang otherwise fuses a multiply and an
// add, even __fmul_rn/__fadd_rn from the HIP headers, into v_fma_f32).
//   momentum: M <- fl32(fl32(mu * M) + G)
__device__ __forceinline__ float momentum_op(float m, float g, float mu) {
#pragma clang fp contract(off)
  const float scaled = mu * m;
  return scaled + g;
}
//   update: W' = W - lr * (O + wd * W), as t = wd*W; u = O + t; v = lr*u; W - v
__device__ __forceinline__ float update_op(float w, float o, float lr, float wd) {
#pragma clang fp contract(off)
  const float t = wd * w;
  const float u = o + t;
  const float v = lr * u;
  return w - v;
}

// The low part of a value v carried as a (bf16 high part h, int8 code q)
// pair.  q counts steps of 256 in v's binary32 bit pattern from h's, and the
// pair decodes to the float whose bits are (h << 16) + 256 q.  h = bf16(v)
// (round to nearest) has v's sign, and floats of one sign are ordered like
// their bit patterns, which are evenly spaced within a binade, so
// |bits(v) - (h << 16)| <= 2^15 (half a bf16 ulp; also when h is the next
// power of two) and the decoded value is within 128 binary32 ulps of v
// (2^-16 relative): about 16 significant bits together.  hs = h << 16, the
// high part's bits as a binary32.  Inf stays inf; NaN decodes to a NaN.
__device__ __forceinline__ uint32_t hi_bits(uint32_t packed, int k) {  // k-th bf16 of a dword, << 16
  return k ? (packed & 0xffff0000u) : (packed << 16);
}
__device__ __forceinline__ int32_t enc_lo(float v, uint32_t hs) {
  const int32_t d = static_cast<int32_t>(__float_as_uint(v) - hs + 128u) >> 8;
  return min(max(d, -128), 127);
}
__device__ __forceinline__ float dec_x(int32_t q, uint32_t hs) {
  return __uint_as_float(hs + (static_cast<uint32_t>(q) << 8));
}
// 4 codes in one dword (byte k = element k) and back
__device__ __forceinline__ uint32_t pack_i8x4(int32_t a, int32_t b, int32_t c, int32_t d) {
  return (static_cast<uint32_t>(a) & 0xff) | ((static_cast<uint32_t>(b) & 0xff) << 8) |
         ((static_cast<uint32_t>(c) & 0xff) << 16) | (static_cast<uint32_t>(d) << 24);
}
__device__ __forceinline__ int32_t i8_at(uint32_t w, int k) {
  return static_cast<int32_t>(static_cast<int8_t>((w >> (8 * k)) & 0xff));
}

// Float atomic max through integer atomics (exact and order-independent): for
// x >= 0 the signed-int order of the bits is the float order; for x < 0 the
// unsigned order is the reverse of it.  NaN is skipped, tested on the bits so
// the test holds in files compiled without NaN semantics for float compares.
__device__ __forceinline__ void atomic_max_float(float* addr, float x) {
  if ((__float_as_uint(x) & 0x7fffffffu) > 0x7f800000u) return;
  if (__float_as_int(x) >= 0) atomicMax(reinterpret_cast<int*>(addr), __float_as_int(x));
  else atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(x));
}

// Range checks of debug builds (MC_DEBUG).  MC_GUARD(tag, cond) is true in
// release builds (the check compiles out).  In a debug build a false cond
// sets bit `tag` of the translation unit's flag word and returns false, and
// the guarded access is skipped, so a bad index is reported instead of
// faulting; MC_DEBUG_UNIT(name) defines debug_take_<name>(), which the C ABI
// calls after each entry point's launches (and after a synchronisation) to
// read and clear the word.
#ifdef MC_DEBUG
static __device__ unsigned int mc_debug_flags;
__device__ __forceinline__ bool mc_guard(bool ok, unsigned int tag) {
  if (!ok) atomicOr(&mc_debug_flags, 1u << tag);
  return ok;
}
#define MC_GUARD(tag, cond) ::mc::mc_guard((cond), (tag))
#define MC_DEBUG_UNIT(name)                                                         \
  unsigned int debug_take_##name() {                                                \
    unsigned int v = 0, z = 0;                                                      \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(mc_debug_flags), sizeof v) != hipSuccess) \
      return 0x80000000u;                                                           \
    if (hipMemcpyToSymbol(HIP_SYMBOL(mc_debug_flags), &z, sizeof z) != hipSuccess)   \
      return 0x80000000u;                                                           \
    return v;                                                                       \
  }
#else
#define MC_GUARD(tag, cond) true
#define MC_DEBUG_UNIT(name)
#endif

// Layout of the Newton-Schulz state X (n_pad x m_pad bf16; its low-part
// codes likewise, one byte per element) in the workspace: column panels of
// 32, each n_pad x 32 row-major (64-byte rows).  A K-step tile of X X^T (256
// rows x 32 columns) is then one contiguous 16 KB run, and a K-rows tile of
// B' X (32 rows x 256 columns) eight contiguous 2 KB runs, so every LDS DMA
// instruction reads 1 KB in one piece.  (Panels of 256 columns, whose rows
// are 512 bytes, made X X^T read 64-byte pieces at a 512-byte pitch: 6-8 %
// slower.)  Element offset of (r, c):
__host__ __device__ __forceinline__ int64_t x_off(int64_t r, int64_t c, int64_t n_pad) {
  return (c >> 5) * n_pad * 32 + r * 32 + (c & 31);
}

// Blocks of one launch are distributed round-robin over the 8 XCDs of an
// MI355X (block b runs on XCD b % 8).  This remap makes consecutive logical
// block ids land on the same XCD, so tiles that share operands share that
// XCD's L2.  Identity when the grid does not divide evenly.
__device__ __forceinline__ uint32_t xcd_grouped_block(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t kXcds = 8;
  if (nblocks % kXcds != 0) return bid;
  return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

}  // namespace mc
