// Internal interface between the C ABI layer (api.cpp) and the kernel
// translation units.  Every launcher enqueues on `stream` and returns the
// hipError_t of the launch; argument checking has already been done by the
// ABI layer, so launchers assume valid, non-empty shapes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mc {

#ifdef MC_DEBUG
// Range-check flags of each kernel unit (debug builds; read and cleared)
unsigned int debug_take_ns_gemm();
unsigned int debug_take_ns_prep();
unsigned int debug_take_qkclip();
unsigned int debug_take_maxlogit();
unsigned int debug_take_attention();
#endif

// ---------------------------------------------------------------- momentum
hipError_t launch_momentum(float* M, const float* G, int64_t numel, float mu, hipStream_t stream);

// ---------------------------------------------------------------- update
// w_bf16/o_bf16 select bfloat16 (true) or float32 (false) storage.
hipError_t launch_update(void* W, bool w_bf16, const void* O, bool o_bf16, int64_t numel, float lr,
                         float weight_decay, hipStream_t stream);

// ---------------------------------------------------------------- Newton-Schulz
// The Muon output scale that matches the update RMS of AdamW:
// sqrt(max(rows, cols)) * 0.2 (Algorithm 1 of "Kimi K2 内部机制"; the Zhihu
// MuonClip formula, "Match Adam Update RMS"), rounded once to float32.
inline float rms_match_scale(int64_t rows, int64_t cols) {
  const double n = static_cast<double>(rows > cols ? rows : cols);
  return static_cast<float>(__builtin_sqrt(n) * 0.2);
}
// out_scale < 0 selects the RMS-matching scale (MC_OUT_SCALE_RMS_MATCH).
inline float resolve_out_scale(float out_scale, int64_t rows, int64_t cols) {
  return out_scale < 0.0f ? rms_match_scale(rows, cols) : out_scale;
}
// Padded internal geometry of one batch of matrices.  X is n x m with
// n = min(rows, cols), m = max(rows, cols); both are padded to multiples of
// the GEMM tile so no kernel needs a bounds check.  Padding is zero, which the
// polynomial keeps zero.
struct NsGeometry {
  int64_t batch, rows, cols;
  int64_t n, m;          // logical
  int64_t n_pad, m_pad;  // padded to kNsTile
  bool transposed;       // rows > cols: X = M^T
  int64_t prescale_tiles;  // 4096-element blocks per matrix of the pre-scale (norm partials)
  // byte offsets inside the workspace: X as bf16 high parts and int8 low-part
  // codes (two ping-pong copies of each, n_pad x m_pad), A and B (n_pad x n_pad), B's
  // diagonal (float32, n_pad), norm partials, 1/norm
  size_t off_x0, off_x1, off_xl0, off_xl1, off_a, off_b, off_d, off_partials, off_invnorm, total;
};
constexpr int64_t kNsTile = 256;
NsGeometry ns_geometry(int64_t batch, int64_t rows, int64_t cols);

// X_0 = M_b unscaled as a (high, low) pair, high part bf16(M) at off_x0 and
// the low part's int8 codes at off_xl0 (M only read, float32 or bf16, batch
// matrices of rows x cols at m_batch_stride), and 1 / (||M_b||_F + eps) per
// matrix at off_invnorm (applied by the first step's GEMMs).
hipError_t launch_ns_prescale_unscaled(const void* M, bool m_bf16, int64_t m_batch_stride, const NsGeometry& g,
                                       float eps, char* ws, hipStream_t stream);
// Fused: M <- mu M + G in place (float32, batch matrices of rows x cols at
// batch_stride), X_0 = M unscaled as a (bf16, int8 code) pair at off_x0 / off_xl0, and
// 1 / (||M||_F + eps) per matrix at off_invnorm (to be applied by the first
// step's GEMMs).
hipError_t launch_momentum_prescale(float* M, const float* G, int64_t batch_stride, float mu,
                                    const NsGeometry& g, float eps, char* ws, hipStream_t stream);
// In-place update applied by the last step's X' = B' X instead of storing X':
// W_b <- W_b - lr * (out_scale * X'_b (transposed back for a tall matrix) +
// wd * W_b), W_b rows x cols at W + b * w_stride, float32 or bf16.  With
// output set, W_b <- out_scale * X'_b instead (W is then the output O, only
// written; lr and wd unused).
struct NsUpdate {
  void* W;
  bool w_bf16;
  int64_t w_stride;
  float out_scale, lr, wd;
  bool output;
};
// One GEMM of the polynomial step, on the whole batch.  X is carried as
// X = Xh + Xl: a bf16 high part and the rounding residual as int8 codes,
// and B = b A + c A A as its float32 diagonal d and a bf16 matrix N with a
// zero diagonal; the products read the high part of X only:
//   mode 0: A = Xh Xh^T                          (in0: Xh, out: A)
//   mode 1: B = alpha A + beta A A               (in0: A, out: N, dg: d)
//   mode 2: X' = a X + d Xh + N Xh, a = `a`      (in0: N, in1: Xh, xl: Xl, dg: d;
//           out: X'h, xl_out: X'l, or the update / output through upd)
// inv (device, per matrix, or null): X is inv_b times the stored X (the first
// step); mode 0 scales A by inv_b^2, mode 2 X' by inv_b.
hipError_t launch_ns_gemm(int mode, const NsGeometry& g, const uint16_t* in0, const uint16_t* in1,
                          const uint8_t* xl, uint16_t* out, uint8_t* xl_out, float* dg, float alpha, float beta,
                          float a, const float* inv, const NsUpdate* upd, hipStream_t stream);

// ---------------------------------------------------------------- max logit
hipError_t launch_maxlogit_init(float* smax, int64_t H, hipStream_t stream);
// Returns hipErrorInvalidValue if no kernel covers the shape (caller checked).
hipError_t launch_maxlogit(const void* Q, const void* Kc, const void* Kr, bool bf16, int64_t B,
                           int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                           hipStream_t stream);
// The float32 LDS-tiled kernel (maxlogit_generic.hip, built with NaN
// semantics) for shapes the MFMA kernel does not cover; scale = 1/sqrt(d).
hipError_t launch_maxlogit_generic(const void* Q, const void* Kc, const void* Kr, bool bf16, int64_t B,
                                   int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                                   float scale, hipStream_t stream);

// ------------------------------------------------------ attention forward
bool attention_fwd_supported(int64_t d_c, int64_t d_r, int64_t d_v);
hipError_t launch_attention_fwd(const void* Q, const void* Kc, const void* Kr, const void* V, int64_t B,
                                int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, int64_t d_v,
                                bool causal, void* O, float* lse, float* smax, hipStream_t stream);

// ---------------------------------------------------------------- QK-Clip
// Layers per launch (their W_q / W_k pointers travel in the kernel arguments).
constexpr int kClipMaxLayers = 64;
// smax [L, H]; Wq / Wk host arrays of L (<= kClipMaxLayers) device pointers;
// gamma_out / clipped_out [L, H] or null.  total_clip requires L == 1.
hipError_t launch_qk_clip(const float* smax, int64_t L, int64_t H, bool total_clip, float tau, float alpha,
                          void* const* Wq, void* const* Wk, bool w_bf16, int64_t d_in, int64_t qph, int64_t q_c_rows,
                          int64_t kph, float* gamma_out, int32_t* clipped_out, hipStream_t stream);

// Measurement aids (probe.hip).
hipError_t launch_mfma_probe(int64_t workgroups, int64_t iters, bool zero_operands, float* out, hipStream_t stream);
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace mc
