// QK-Clip: per-head rescale of the query/key projection rows.
//
// For a head h with S_max^h > tau, gamma = tau / S_max^h (computed on the
// device: no host round trip per head), and in place
//   W_q rows of the head's first q_c_rows       x gamma^alpha
//   W_q rows of the rest of the head             x gamma
//   W_k rows of the head                         x gamma^(1 - alpha)
// ("Kimi K2 内部机制", MuonClip section: per-head gamma_h = min(1, tau/S_max^h),
// W_q^h by gamma^alpha and W_k^h by gamma^(1-alpha), and the MLA table that
// scales q^C and k^C by sqrt(gamma), q^R by gamma and leaves the shared k^R).
//
// Total clip (the variant the same section describes before per-head clip):
// one gamma = tau / S_max from S_max = max_h S_max^h (NaN heads skipped; all
// NaN leaves everything untouched), applied to every head with the same
// split when S_max > tau.  Each block reduces the H values itself.
//
// Several attention layers (the pages clip every head of every attention
// layer) go in one launch: S_max is [L, H] row-major, layer l's W_q / W_k
// come from a table of L pointers in the kernel arguments, and "head" below
// means one of the L x H (layer, head) pairs.  A head's rows are two
// contiguous row blocks (W_q and W_k are row-major with head-major rows), so
// the kernels stream them with 16-byte accesses.  Compact kernel (up to 4000
// heads): every block reads all L x H values of S_max, lists the clipped
// heads with their factors in LDS (16 bytes per head), and the grid, sized for the case where
// every head is clipped, shares out only the listed heads' elements, so few
// clipped heads still spread over every CU and no block is launched just to
// find its head unclipped.  More heads: a grid of (chunks, L x H) whose
// blocks of unclipped heads return after reading one float.
//
// The multiply is a single float op, rounded once to the storage type; FP
// contraction is off so the result does not depend on the compiler.

#include <math.h>

#include "mc_device.h"
#include "mc_internal.h"

namespace mc {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;  // 16-byte vectors per thread per block

// W_q / W_k of each layer of one launch
struct LayerPtrs {
  void* q[kClipMaxLayers];
  void* k[kClipMaxLayers];
};

struct ClipFactors {
  float q_c, q_r, k;
  int32_t state;  // 1 clipped, 0 not, -1 NaN
  float gamma;
};

__device__ __forceinline__ ClipFactors clip_factors(float s, float tau, float alpha) {
  ClipFactors f;
  if (s != s) {
    f = {1.f, 1.f, 1.f, -1, 1.f};
  } else if (s > tau) {  // strict: a head exactly at tau is not touched
    const float g = tau / s;
    float qa, ka;
    if (alpha == 0.5f) {
      qa = sqrtf(g);
      ka = qa;
    } else {
      qa = powf(g, alpha);
      ka = powf(g, 1.0f - alpha);
    }
    f = {qa, g, ka, 1, g};
  } else {
    f = {1.f, 1.f, 1.f, 0, 1.f};
  }
  return f;
}

__device__ __forceinline__ float scale_op(float w, float f) {
#pragma clang fp contract(off)
  return w * f;
}

template <bool BF16>
__device__ __forceinline__ void scale_vec8(void* base, int64_t v, float f) {
  if constexpr (BF16) {
    u32x4* p = reinterpret_cast<u32x4*>(base) + v;
    u32x4 a = *p;
    a.x = pack_bf16x2(scale_op(bf16_lo(a.x), f), scale_op(bf16_hi(a.x), f));
    a.y = pack_bf16x2(scale_op(bf16_lo(a.y), f), scale_op(bf16_hi(a.y), f));
    a.z = pack_bf16x2(scale_op(bf16_lo(a.z), f), scale_op(bf16_hi(a.z), f));
    a.w = pack_bf16x2(scale_op(bf16_lo(a.w), f), scale_op(bf16_hi(a.w), f));
    *p = a;
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(base) + 2 * v;
    f32x4 a = p[0], b = p[1];
    a.x = scale_op(a.x, f); a.y = scale_op(a.y, f); a.z = scale_op(a.z, f); a.w = scale_op(a.w, f);
    b.x = scale_op(b.x, f); b.y = scale_op(b.y, f); b.z = scale_op(b.z, f); b.w = scale_op(b.w, f);
    p[0] = a;
    p[1] = b;
  }
}

template <bool BF16>
__device__ __forceinline__ void scale_one(void* base, int64_t i, float f) {
  if constexpr (BF16) {
    uint16_t* p = static_cast<uint16_t*>(base) + i;
    *p = f32_to_bf16(scale_op(bf16_to_f32(*p), f));
  } else {
    float* p = static_cast<float*>(base) + i;
    *p = scale_op(*p, f);
  }
}

// max over smax[0 .. H) skipping NaNs (NaN only if all are NaN), the same
// value in every thread of the block
__device__ float block_max_all(const float* __restrict__ smax, int64_t H) {
  __shared__ float red[kThreads / 64];
  float m = __builtin_nanf("");
  for (int64_t i = threadIdx.x; i < H; i += kThreads) m = fmaxf(m, smax[i]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

// VEC: every row block starts 16-byte aligned and d_in % 8 == 0, so the
// element ranges below are whole 8-element vectors.  total_clip (one layer):
// one gamma from the largest S_max of all heads.  grid (chunks, L * H).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void qk_clip_kernel(const float* __restrict__ smax, int64_t H, bool total_clip,
                                                          float tau, float alpha, LayerPtrs lp, int64_t d_in,
                                                          int64_t qph, int64_t q_c_rows, int64_t kph,
                                                          float* __restrict__ gamma_out,
                                                          int32_t* __restrict__ clipped_out) {
  const int64_t gh = blockIdx.y, layer = gh / H, h = gh - layer * H;
  const ClipFactors f = clip_factors(total_clip ? block_max_all(smax, H) : smax[gh], tau, alpha);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (gamma_out) gamma_out[gh] = f.gamma;
    if (clipped_out) clipped_out[gh] = f.state;
  }
  if (f.state != 1) return;

  const size_t esz = BF16 ? 2 : 4;
  char* q_base = static_cast<char*>(lp.q[layer]) + static_cast<size_t>(h * qph * d_in) * esz;
  char* k_base = static_cast<char*>(lp.k[layer]) + static_cast<size_t>(h * kph * d_in) * esz;
  const int64_t q_elems = qph * d_in, q_c_elems = q_c_rows * d_in, k_elems = kph * d_in;
  const int64_t total = q_elems + k_elems;

  if constexpr (VEC) {
    const int64_t nvec = total / 8, q_vec = q_elems / 8, q_c_vec = q_c_elems / 8;
    const int64_t per_block = static_cast<int64_t>(kThreads) * kVecPerThread;
    const int64_t v_end = min(nvec, (static_cast<int64_t>(blockIdx.x) + 1) * per_block);
    for (int64_t v = blockIdx.x * per_block + threadIdx.x; v < v_end; v += kThreads) {
      if (v < q_vec) scale_vec8<BF16>(q_base, v, v < q_c_vec ? f.q_c : f.q_r);
      else scale_vec8<BF16>(k_base, v - q_vec, f.k);
    }
  } else {
    const int64_t per_block = static_cast<int64_t>(kThreads) * kVecPerThread * 8;
    const int64_t e_end = min(total, (static_cast<int64_t>(blockIdx.x) + 1) * per_block);
    for (int64_t e = blockIdx.x * per_block + threadIdx.x; e < e_end; e += kThreads) {
      if (e < q_elems) scale_one<BF16>(q_base, e, e < q_c_elems ? f.q_c : f.q_r);
      else scale_one<BF16>(k_base, e - q_elems, f.k);
    }
  }
}


constexpr int kCompactMaxHeads = 4000;  // heads per layer; the list then takes at most 64000 bytes of LDS
constexpr int kCompactMaxBlocks = 4096;

// grid (blocks per layer, L).  Block (x, l) lists layer l's clipped heads
// (identical in every block of the layer) with their factors in dynamic LDS
// sized for H entries (16 bytes each), then takes share x of that layer's
// clipped elements; block (0, l) also writes gamma_out / clipped_out of the
// layer's heads.  total_clip: one layer, gamma from the largest S_max.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void qk_clip_compact_kernel(const float* __restrict__ smax_all, int H,
                                                                  bool total_clip, float tau, float alpha,
                                                                  LayerPtrs lp, int64_t d_in, int64_t qph,
                                                                  int64_t q_c_rows, int64_t kph,
                                                                  float* __restrict__ gamma_out,
                                                                  int32_t* __restrict__ clipped_out) {
  extern __shared__ __attribute__((aligned(16))) char clip_list[];
  int* l_head = reinterpret_cast<int*>(clip_list);
  float* l_qc = reinterpret_cast<float*>(clip_list) + H;
  float* l_qr = l_qc + H;
  float* l_k = l_qr + H;
  __shared__ int wave_count[kThreads / 64];
  const int layer = blockIdx.y;
  const float* smax = smax_all + static_cast<int64_t>(layer) * H;
  const float s_all = total_clip ? block_max_all(smax, H) : 0.0f;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int count = 0;  // the same in every thread
  for (int base = 0; base < H; base += kThreads) {
    const int h = base + static_cast<int>(threadIdx.x);
    ClipFactors f = {1.f, 1.f, 1.f, 0, 1.f};
    if (h < H) f = clip_factors(total_clip ? s_all : smax[h], tau, alpha);
    if (blockIdx.x == 0 && h < H) {
      if (gamma_out) gamma_out[static_cast<int64_t>(layer) * H + h] = f.gamma;
      if (clipped_out) clipped_out[static_cast<int64_t>(layer) * H + h] = f.state;
    }
    const bool c = h < H && f.state == 1;
    const uint64_t m = __ballot(c);
    if (lane == 0) wave_count[w] = __popcll(m);
    __syncthreads();
    int slot = count + __popcll(m & ((uint64_t{1} << lane) - 1));
    int round = 0;
    for (int i = 0; i < kThreads / 64; ++i) {
      if (i < w) slot += wave_count[i];
      round += wave_count[i];
    }
    if (c && MC_GUARD(0, slot < H)) {
      l_head[slot] = h;
      l_qc[slot] = f.q_c;
      l_qr[slot] = f.q_r;
      l_k[slot] = f.k;
    }
    count += round;
    __syncthreads();
  }
  if (count == 0) return;
  char* const q_layer = static_cast<char*>(lp.q[layer]);
  char* const k_layer = static_cast<char*>(lp.k[layer]);

  const size_t esz = BF16 ? 2 : 4;
  const int64_t unit = VEC ? 8 : 1;  // elements per work item
  const int64_t q_items = qph * d_in / unit, q_c_items = q_c_rows * d_in / unit;
  const int64_t per_head = q_items + kph * d_in / unit;
  const int64_t total = count * per_head;
  // Work items go out in batches of kUnroll x kThreads consecutive items (a
  // thread's kUnroll items kThreads apart), block x taking batches x,
  // x + gridDim.x, ..., so the blocks of a layer sweep adjacent memory
  // together (one contiguous range per block ran 12 % slower on all 64
  // heads: scattered DRAM rows); a batch's loads are all issued before any
  // item is scaled and stored, so kUnroll 16-byte loads per thread are in
  // flight at once, and the accesses are non-temporal (each element is
  // touched once).  The head of an item follows from the batch's first head
  // without a division per item.
  constexpr int kUnroll = 4;
  constexpr int64_t kBatch = static_cast<int64_t>(kUnroll) * kThreads;
  const int64_t v_end = total;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kBatch; base < v_end;
       base += static_cast<int64_t>(gridDim.x) * kBatch) {
    const int idx0 = static_cast<int>(base / per_head);
    char* addr[kUnroll];
    float fac[kUnroll];
    constexpr int kWords = VEC && !BF16 ? 2 : 1;  // 16-byte words per item
    u32x4 val[kUnroll][kWords];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = base + u * kThreads + threadIdx.x;
      addr[u] = nullptr;
      if (v >= v_end) continue;
      int idx = idx0;
      int64_t off = v - static_cast<int64_t>(idx0) * per_head;
      while (off >= per_head) {
        off -= per_head;
        ++idx;
      }
      if (!MC_GUARD(1, idx < count)) continue;
      const int64_t h = l_head[idx];
      const bool in_q = off < q_items;
      char* row_base = in_q ? q_layer + static_cast<size_t>(h * qph * d_in) * esz
                            : k_layer + static_cast<size_t>(h * kph * d_in) * esz;
      const int64_t o = in_q ? off : off - q_items;
      fac[u] = in_q ? (off < q_c_items ? l_qc[idx] : l_qr[idx]) : l_k[idx];
      if (!MC_GUARD(2, h < H && o >= 0 && (o + 1) * unit <= (in_q ? qph : kph) * d_in)) continue;
      addr[u] = row_base + static_cast<size_t>(o * unit) * esz;
      if constexpr (VEC) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) val[u][w] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(addr[u]) + w);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (addr[u] == nullptr) continue;
      if constexpr (VEC) {
        if constexpr (BF16) {
          u32x4 a = val[u][0];
          const float f = fac[u];
          a.x = pack_bf16x2(scale_op(bf16_lo(a.x), f), scale_op(bf16_hi(a.x), f));
          a.y = pack_bf16x2(scale_op(bf16_lo(a.y), f), scale_op(bf16_hi(a.y), f));
          a.z = pack_bf16x2(scale_op(bf16_lo(a.z), f), scale_op(bf16_hi(a.z), f));
          a.w = pack_bf16x2(scale_op(bf16_lo(a.w), f), scale_op(bf16_hi(a.w), f));
          __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(addr[u]));
        } else {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            f32x4 a = __builtin_bit_cast(f32x4, val[u][w % kWords]);
            a.x = scale_op(a.x, fac[u]); a.y = scale_op(a.y, fac[u]);
            a.z = scale_op(a.z, fac[u]); a.w = scale_op(a.w, fac[u]);
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, a), reinterpret_cast<u32x4*>(addr[u]) + w);
          }
        }
      } else {
        scale_one<BF16>(addr[u], 0, fac[u]);
      }
    }
  }
}
}  // namespace

MC_DEBUG_UNIT(qkclip)

hipError_t launch_qk_clip(const float* smax, int64_t L, int64_t H, bool total_clip, float tau, float alpha,
                          void* const* Wq, void* const* Wk, bool w_bf16, int64_t d_in, int64_t qph, int64_t q_c_rows,
                          int64_t kph, float* gamma_out, int32_t* clipped_out, hipStream_t stream) {
  const size_t esz = w_bf16 ? 2 : 4;
  LayerPtrs lp{};
  bool vec = (d_in % 8 == 0) && ((qph * d_in * static_cast<int64_t>(esz)) % 16 == 0) &&
             ((kph * d_in * static_cast<int64_t>(esz)) % 16 == 0);
  for (int64_t l = 0; l < L; ++l) {
    lp.q[l] = Wq[l];
    lp.k[l] = Wk[l];
    vec = vec && reinterpret_cast<uintptr_t>(Wq[l]) % 16 == 0 && reinterpret_cast<uintptr_t>(Wk[l]) % 16 == 0;
  }
  const int64_t NH = L * H;
  const int64_t total = (qph + kph) * d_in;
  if (H <= kCompactMaxHeads) {
    // blocks per layer for every head clipped: one work item per thread, at
    // most kCompactMaxBlocks blocks over all layers (then each thread loops)
    const int64_t items = H * (vec ? total / 8 : total);
    int64_t blocks = (items + kThreads - 1) / kThreads;
    const int64_t cap = kCompactMaxBlocks / L > 0 ? kCompactMaxBlocks / L : 1;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
#define MC_CLIP_COMPACT(B, V)                                                                                     \
  hipLaunchKernelGGL((qk_clip_compact_kernel<B, V>), dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(L)), \
                     dim3(kThreads), static_cast<unsigned>(H * 16), stream, smax, static_cast<int>(H), total_clip,   \
                     tau, alpha, lp, d_in, qph, q_c_rows, kph, gamma_out, clipped_out)
    if (w_bf16) {
      if (vec) MC_CLIP_COMPACT(true, true);
      else MC_CLIP_COMPACT(true, false);
    } else {
      if (vec) MC_CLIP_COMPACT(false, true);
      else MC_CLIP_COMPACT(false, false);
    }
#undef MC_CLIP_COMPACT
    return hipGetLastError();
  }
  const int64_t per_block = static_cast<int64_t>(kThreads) * kVecPerThread * 8;
  int64_t chunks = (total + per_block - 1) / per_block;
  if (chunks < 1) chunks = 1;
  dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(NH));
#define MC_CLIP_LAUNCH(B, V)                                                                   \
  hipLaunchKernelGGL((qk_clip_kernel<B, V>), grid, dim3(kThreads), 0, stream, smax, H, total_clip, tau, alpha, \
                     lp, d_in, qph, q_c_rows, kph, gamma_out, clipped_out)
  if (w_bf16) {
    if (vec) MC_CLIP_LAUNCH(true, true);
    else MC_CLIP_LAUNCH(true, false);
  } else {
    if (vec) MC_CLIP_LAUNCH(false, true);
    else MC_CLIP_LAUNCH(false, false);
  }
#undef MC_CLIP_LAUNCH
  return hipGetLastError();
}

}  // namespace mc
