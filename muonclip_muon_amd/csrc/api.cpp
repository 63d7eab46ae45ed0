// C ABI of libmuonclip.so: argument validation and dispatch to the kernels.
// Every check runs before anything is enqueued, so an invalid call touches
// no output; see include/muonclip.h for the contract of each entry point.

#include "muonclip.h"
#include "muonclip_probe.h"

#include <math.h>
#include <stdio.h>

#include <initializer_list>
#include <mutex>
#include <utility>

#include "mc_internal.h"

namespace {

inline bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
inline bool valid_dtype(int d) { return d == MC_F32 || d == MC_BF16; }
inline size_t dtype_size(int d) { return d == MC_BF16 ? 2 : 4; }
inline mc_status_t from_hip(hipError_t e) { return e == hipSuccess ? MC_OK : MC_EHIP; }

// The status of an entry point whose launches returned e.  Debug builds
// (MC_DEBUG) also wait for the stream and read every kernel unit's
// range-check flags; failed checks are printed and returned as MC_ECHECK.
mc_status_t done(hipError_t e, void* stream, const char* fn) {
  if (e != hipSuccess) return MC_EHIP;
#ifdef MC_DEBUG
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return MC_EHIP;
  struct Unit {
    const char* name;
    unsigned int (*take)();
  };
  const Unit units[] = {{"ns_gemm", mc::debug_take_ns_gemm}, {"ns_prep", mc::debug_take_ns_prep},
                        {"qkclip", mc::debug_take_qkclip},   {"maxlogit", mc::debug_take_maxlogit},
                        {"attention", mc::debug_take_attention}};
  unsigned int failed = 0;
  for (const Unit& u : units) {
    const unsigned int v = u.take();
    if (v != 0) fprintf(stderr, "libmuonclip (debug): %s: range checks 0x%x failed in %s\n", fn, v, u.name);
    failed |= v;
  }
  if (failed != 0) return MC_ECHECK;
#else
  (void)stream;
  (void)fn;
#endif
  return MC_OK;
}

constexpr int64_t kNsMaxN = 16384;   // min(rows, cols)
constexpr int64_t kNsMaxM = 65536;   // max(rows, cols)
constexpr int32_t kNsMaxSteps = 64;
constexpr int64_t kGridMax = 0x7fffffff;

// A product of non-negative sizes no larger than 2^46 (far beyond any
// buffer a GPU holds), computed without overflow: sizes whose element counts
// or offsets could leave int64 are rejected before any is formed.
inline bool count_ok(std::initializer_list<int64_t> dims) {
  __int128 p = 1;
  for (int64_t d : dims) {
    if (d < 0) return false;
    p *= d;
    if (p > (static_cast<__int128>(1) << 46)) return false;
  }
  return true;
}

// The batch limits of the Newton-Schulz calls (grid sizes), checked before
// any size is computed from the batch: at most 65535 matrices (the
// pre-scale's grid z) and fewer than 2^31 GEMM tiles in one launch.
inline bool ns_batch_supported(int64_t batch, int64_t n, int64_t m) {
  const int64_t tiles = ((n + 255) / 256) * ((m + 255) / 256);
  return batch <= 65535 && tiles * batch <= kGridMax;
}

}  // namespace

extern "C" {

int mc_abi_version(void) { return MC_ABI_VERSION; }

int mc_debug_build(void) {
#ifdef MC_DEBUG
  return 1;
#else
  return 0;
#endif
}

const char* mc_status_string(int status) {
  switch (status) {
    case MC_OK: return "ok";
    case MC_EINVAL: return "invalid argument";
    case MC_ESHAPE: return "unsupported shape";
    case MC_EDTYPE: return "unsupported dtype";
    case MC_EALIGN: return "misaligned pointer";
    case MC_EWORKSPACE: return "workspace missing or too small";
    case MC_EHIP: return "HIP runtime error";
    case MC_ECHECK: return "range check failed (debug build)";
    default: return "unknown status";
  }
}

mc_status_t muonclip_momentum(float* M, const float* G, int64_t numel, float mu, void* stream) {
  if (numel < 0) return MC_EINVAL;
  if (numel == 0) return MC_OK;
  if (!M || !G) return MC_EINVAL;
  if (!isfinite(mu)) return MC_EINVAL;
  if (!aligned(M, 4) || !aligned(G, 4)) return MC_EALIGN;
  return done(mc::launch_momentum(M, G, numel, mu, static_cast<hipStream_t>(stream)), stream, __func__);
}

float muon_rms_match_scale(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1) return 0.0f;
  return mc::rms_match_scale(rows, cols);
}

size_t muon_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 0 || rows < 1 || cols < 1) return 0;
  const int64_t n = rows < cols ? rows : cols, m = rows < cols ? cols : rows;
  if (n > kNsMaxN || m > kNsMaxM || !ns_batch_supported(batch, n, m)) return 0;
  return mc::ns_geometry(batch, rows, cols).total;
}

}  // extern "C"

namespace {

// Checks shared by the Newton-Schulz entry points (shape, steps, coefficients,
// eps, scale, workspace, events); fills g on success.
mc_status_t check_ns(int64_t batch, int64_t rows, int64_t cols, int32_t steps, const float* coeffs, float eps,
                     float out_scale, void* workspace, size_t workspace_bytes, void* const* gemm_events,
                     mc::NsGeometry* g) {
  const int64_t n = rows < cols ? rows : cols, m = rows < cols ? cols : rows;
  if (n > kNsMaxN || m > kNsMaxM || !ns_batch_supported(batch, n, m)) return MC_ESHAPE;
  if (!coeffs || !workspace) return MC_EINVAL;
  if (steps < 1 || steps > kNsMaxSteps) return MC_EINVAL;
  if (!(eps >= 0.0f) || !isfinite(eps) || !isfinite(out_scale)) return MC_EINVAL;
  for (int i = 0; i < 3 * steps; ++i)
    if (!isfinite(coeffs[i])) return MC_EINVAL;
  if (!aligned(workspace, 256)) return MC_EALIGN;
  *g = mc::ns_geometry(batch, rows, cols);
  if (workspace_bytes < g->total) return MC_EWORKSPACE;
  if (gemm_events)
    for (int i = 0; i < 6 * steps; ++i)
      if (!gemm_events[i]) return MC_EINVAL;
  return MC_OK;
}

// The steps' GEMMs, X_0 at off_x0 (high part) and off_xl0 (low part):
// A = Xh Xh^T; B = b A + c A A = diag(d) + N; X <- a X + d Xh + N Xh (X
// carried as bf16 high parts and int8 low-part codes, d in float32).
// inv0 (or null): the stored X_0 is to be scaled per matrix by inv0 (applied
// inside the first step).  upd (or null): the last step updates W (or writes
// the output) instead of storing X.
hipError_t run_ns_steps(const mc::NsGeometry& g, char* ws, int32_t steps, const float* coeffs, const float* inv0,
                        const mc::NsUpdate* upd, hipStream_t s, void* const* gemm_events) {
  uint16_t* X = reinterpret_cast<uint16_t*>(ws + g.off_x0);
  uint16_t* Xn = reinterpret_cast<uint16_t*>(ws + g.off_x1);
  uint8_t* XL = reinterpret_cast<uint8_t*>(ws + g.off_xl0);
  uint8_t* XLn = reinterpret_cast<uint8_t*>(ws + g.off_xl1);
  uint16_t* A = reinterpret_cast<uint16_t*>(ws + g.off_a);
  uint16_t* B = reinterpret_cast<uint16_t*>(ws + g.off_b);
  float* D = reinterpret_cast<float*>(ws + g.off_d);
  auto record = [&](int idx) -> hipError_t {
    return gemm_events ? hipEventRecord(static_cast<hipEvent_t>(gemm_events[idx]), s) : hipSuccess;
  };
  hipError_t e = hipSuccess;
  for (int st = 0; st < steps; ++st) {
    const float a = coeffs[3 * st], b = coeffs[3 * st + 1], c = coeffs[3 * st + 2];
    const float* inv = st == 0 ? inv0 : nullptr;
    const bool last = st == steps - 1;
    for (int gm = 0; gm < 3; ++gm) {
      if ((e = record(2 * (3 * st + gm))) != hipSuccess) return e;
      if (gm == 0)
        e = mc::launch_ns_gemm(0, g, X, nullptr, nullptr, A, nullptr, nullptr, 0.f, 0.f, 0.f, inv, nullptr, s);
      else if (gm == 1)
        e = mc::launch_ns_gemm(1, g, A, nullptr, nullptr, B, nullptr, D, b, c, 0.f, nullptr, nullptr, s);
      else
        e = mc::launch_ns_gemm(2, g, B, X, XL, Xn, XLn, D, 0.f, 0.f, a, inv, last ? upd : nullptr, s);
      if (e != hipSuccess) return e;
      if ((e = record(2 * (3 * st + gm) + 1)) != hipSuccess) return e;
    }
    std::swap(X, Xn);
    std::swap(XL, XLn);
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

mc_status_t muon_ns_orthogonalize_batched(const void* M, int m_dtype, int64_t batch, int64_t rows,
                                          int64_t cols, int64_t m_batch_stride, void* O, int o_dtype,
                                          int64_t o_batch_stride, int32_t steps, const float* coeffs,
                                          float eps, float out_scale, void* workspace,
                                          size_t workspace_bytes, void* stream,
                                          void* const* gemm_events) {
  if (batch < 0 || rows < 1 || cols < 1) return MC_EINVAL;
  if (!valid_dtype(m_dtype) || !valid_dtype(o_dtype)) return MC_EDTYPE;
  {
    const int64_t n = rows < cols ? rows : cols, m = rows < cols ? cols : rows;
    if (n > kNsMaxN || m > kNsMaxM) return MC_ESHAPE;
  }
  if (batch == 0) return MC_OK;
  if (!M || !O) return MC_EINVAL;
  if (batch > 1 && (m_batch_stride < rows * cols || o_batch_stride < rows * cols)) return MC_EINVAL;
  if (!aligned(M, dtype_size(m_dtype)) || !aligned(O, dtype_size(o_dtype))) return MC_EALIGN;
  mc::NsGeometry g;
  const mc_status_t st = check_ns(batch, rows, cols, steps, coeffs, eps, out_scale, workspace, workspace_bytes,
                                  gemm_events, &g);
  if (st != MC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool m_bf16 = m_dtype == MC_BF16, o_bf16 = o_dtype == MC_BF16;
  // X_0 = bf16(M) unscaled plus 1 / (||M||_F + eps), applied by the first
  // step's GEMM epilogues, as in the fused call
  if (mc::launch_ns_prescale_unscaled(M, m_bf16, m_batch_stride, g, eps, ws, s) != hipSuccess) return MC_EHIP;
  const float* inv = reinterpret_cast<const float*>(ws + g.off_invnorm);
  // the last step's X' = B' X writes O = out_scale * X' (transposed back)
  mc::NsUpdate out{O, o_bf16, o_batch_stride, mc::resolve_out_scale(out_scale, rows, cols), 0.f, 0.f, true};
  return done(run_ns_steps(g, ws, steps, coeffs, inv, &out, s, gemm_events), stream, __func__);
}

}  // extern "C"

namespace {

// The fused Muon call on a given scratch buffer (a caller workspace or the
// library's static scratch); every check runs before anything is enqueued.
mc_status_t fused_muon(float* M, const float* G, float mu, void* W, int w_dtype, int64_t batch, int64_t rows,
                       int64_t cols, int64_t batch_stride, int32_t steps, const float* coeffs, float eps,
                       float out_scale, float lr, float weight_decay, void* workspace, size_t workspace_bytes,
                       void* stream, void* const* gemm_events) {
  if (batch < 0 || rows < 1 || cols < 1) return MC_EINVAL;
  if (!valid_dtype(w_dtype)) return MC_EDTYPE;
  {
    const int64_t n = rows < cols ? rows : cols, m = rows < cols ? cols : rows;
    if (n > kNsMaxN || m > kNsMaxM) return MC_ESHAPE;
  }
  if (batch == 0) return MC_OK;
  if (!M || !G || !W) return MC_EINVAL;
  if (batch > 1 && batch_stride < rows * cols) return MC_EINVAL;
  if (!isfinite(mu) || !isfinite(lr) || !isfinite(weight_decay)) return MC_EINVAL;
  if (!aligned(M, 4) || !aligned(G, 4) || !aligned(W, dtype_size(w_dtype))) return MC_EALIGN;
  mc::NsGeometry g;
  const mc_status_t st = check_ns(batch, rows, cols, steps, coeffs, eps, out_scale, workspace, workspace_bytes,
                                  gemm_events, &g);
  if (st != MC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (mc::launch_momentum_prescale(M, G, batch_stride, mu, g, eps, ws, s) != hipSuccess) return MC_EHIP;
  const float* inv = reinterpret_cast<const float*>(ws + g.off_invnorm);
  mc::NsUpdate upd{W, w_dtype == MC_BF16, batch_stride, mc::resolve_out_scale(out_scale, rows, cols), lr,
                   weight_decay, false};
  return done(run_ns_steps(g, ws, steps, coeffs, inv, &upd, s, gemm_events), stream, "muon_momentum_ns_update_batched");
}

// Scratch of the allocation-free entry point: a file-scope device array, one
// copy per GPU, resident from the library's first use on that GPU until the
// process ends.  The name is a host-side stand-in for the device symbol; its
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = MC_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of `scratch` on the device the kernels of a call on `stream`
// run on (the stream's device; the current device for the null stream),
// looked up on that device's first call with that device made current, or
// null on failure.
void* static_scratch(hipStream_t stream) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
    dev = static_cast<int>(d);
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

mc_status_t muon_momentum_ns_update_batched(float* M, const float* G, float mu, void* W, int w_dtype,
                                            int64_t batch, int64_t rows, int64_t cols, int64_t batch_stride,
                                            int32_t steps, const float* coeffs, float eps, float out_scale,
                                            float lr, float weight_decay, void* workspace,
                                            size_t workspace_bytes, void* stream, void* const* gemm_events) {
  return fused_muon(M, G, mu, W, w_dtype, batch, rows, cols, batch_stride, steps, coeffs, eps, out_scale, lr,
                    weight_decay, workspace, workspace_bytes, stream, gemm_events);
}

mc_status_t muon_momentum_ns_update_batched_noalloc(float* M, const float* G, float mu, void* W, int w_dtype,
                                                    int64_t batch, int64_t rows, int64_t cols,
                                                    int64_t batch_stride, int32_t steps, const float* coeffs,
                                                    float eps, float out_scale, float lr, float weight_decay,
                                                    void* stream) {
  // shape checks first (a size beyond the static scratch is MC_EWORKSPACE;
  // nothing is looked up or enqueued for an invalid call)
  if (batch < 0 || rows < 1 || cols < 1) return MC_EINVAL;
  {
    const int64_t n = rows < cols ? rows : cols, m = rows < cols ? cols : rows;
    if (n > kNsMaxN || m > kNsMaxM) return MC_ESHAPE;
  }
  if (batch == 0) return MC_OK;
  if (!ns_batch_supported(batch, rows < cols ? rows : cols, rows < cols ? cols : rows)) return MC_ESHAPE;
  if (mc::ns_geometry(batch, rows, cols).total > kStaticScratchBytes) return MC_EWORKSPACE;
  void* ws = static_scratch(static_cast<hipStream_t>(stream));
  if (!ws) return MC_EHIP;
  return fused_muon(M, G, mu, W, w_dtype, batch, rows, cols, batch_stride, steps, coeffs, eps, out_scale, lr,
                    weight_decay, ws, kStaticScratchBytes, stream, nullptr);
}

mc_status_t muon_apply_update(void* W, int w_dtype, const void* O, int o_dtype, int64_t numel,
                              float lr, float weight_decay, void* stream) {
  if (numel < 0) return MC_EINVAL;
  if (!valid_dtype(w_dtype) || !valid_dtype(o_dtype)) return MC_EDTYPE;
  if (numel == 0) return MC_OK;
  if (!W || !O) return MC_EINVAL;
  if (!isfinite(lr) || !isfinite(weight_decay)) return MC_EINVAL;
  if (!aligned(W, dtype_size(w_dtype)) || !aligned(O, dtype_size(o_dtype))) return MC_EALIGN;
  return done(mc::launch_update(W, w_dtype == MC_BF16, O, o_dtype == MC_BF16, numel, lr, weight_decay,
                                static_cast<hipStream_t>(stream)),
              stream, __func__);
}

mc_status_t qk_maxlogit(const void* Q, const void* Kc, const void* Kr, int dtype, int64_t B, int64_t H,
                        int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                        int32_t accumulate, void* stream) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || d_c < 1 || d_r < 0) return MC_EINVAL;
  if (!valid_dtype(dtype)) return MC_EDTYPE;
  if (d_c + d_r > 512) return MC_ESHAPE;
  if (H == 0) return MC_OK;
  if (!smax) return MC_EINVAL;
  if (H > 65535 || B > 65535 || (Sq + 63) / 64 > kGridMax) return MC_ESHAPE;
  if (!count_ok({B, H, Sq, d_c + d_r}) || !count_ok({B, H, Sk, d_c}) || !count_ok({B, Sk, d_r}))
    return MC_ESHAPE;
  const bool empty = B == 0 || Sq == 0 || Sk == 0;
  if (!empty) {
    if (!Q || !Kc) return MC_EINVAL;
    if ((d_r > 0) != (Kr != nullptr)) return MC_EINVAL;
    const size_t es = dtype_size(dtype);
    if (!aligned(Q, es) || !aligned(Kc, es) || (Kr && !aligned(Kr, es))) return MC_EALIGN;
  }
  if (!aligned(smax, 4)) return MC_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!accumulate) {
    hipError_t e = mc::launch_maxlogit_init(smax, H, s);
    if (e != hipSuccess) return MC_EHIP;
  }
  if (empty) return MC_OK;
  return done(mc::launch_maxlogit(Q, Kc, Kr, dtype == MC_BF16, B, H, Sq, Sk, d_c, d_r, smax, s), stream, __func__);
}

mc_status_t attention_fwd_maxlogit(const void* Q, const void* Kc, const void* Kr, const void* V, int dtype,
                                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r,
                                   int64_t d_v, int32_t causal, void* O, float* lse_out, float* smax_out,
                                   int32_t accumulate, void* stream) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || d_c < 0 || d_r < 0 || d_v < 0) return MC_EINVAL;
  if (!valid_dtype(dtype)) return MC_EDTYPE;
  if (dtype != MC_BF16) return MC_EDTYPE;
  if (!mc::attention_fwd_supported(d_c, d_r, d_v)) return MC_ESHAPE;
  if (H > 65535 || Sq > INT32_MAX || Sk > INT32_MAX) return MC_ESHAPE;
  if (!count_ok({B, H, Sq, d_c + d_r}) || !count_ok({B, H, Sk, d_c + d_v}) || !count_ok({B, Sk, d_r}) ||
      !count_ok({B, H, Sq, d_v}))
    return MC_ESHAPE;
  // an empty call (no batch, head or query row) reads and writes no tensor
  // but S_max, so only smax_out has to point somewhere (and only for H > 0)
  const bool empty = B == 0 || H == 0 || Sq == 0;
  if (H > 0 && !smax_out) return MC_EINVAL;
  if (!empty && (!Q || !Kc || !V || !O || (d_r > 0 && !Kr))) return MC_EINVAL;
  if (!empty && Sk < 64) return MC_ESHAPE;
  if (causal && Sq > Sk) return MC_ESHAPE;
  if (B * H * ((Sq + 255) / 256) > kGridMax) return MC_ESHAPE;
  if (!aligned(Q, 16) || !aligned(Kc, 16) || (Kr && !aligned(Kr, 16)) || !aligned(V, 16) || !aligned(O, 8) ||
      !aligned(smax_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return MC_EALIGN;
  if (H == 0) return MC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!accumulate) {
    hipError_t e = mc::launch_maxlogit_init(smax_out, H, s);
    if (e != hipSuccess) return MC_EHIP;
  }
  if (empty) return MC_OK;
  return done(mc::launch_attention_fwd(Q, Kc, Kr, V, B, H, Sq, Sk, d_c, d_r, d_v, causal != 0, O, lse_out,
                                       smax_out, s),
              stream, __func__);
}

static mc_status_t qk_clip_check(int64_t H, float tau, float alpha, int w_dtype, int64_t d_in, int64_t q_rows_per_head,
                                 int64_t q_c_rows, int64_t k_rows_per_head) {
  if (H < 0 || d_in < 1 || q_rows_per_head < 0 || q_c_rows < 0 || q_c_rows > q_rows_per_head ||
      k_rows_per_head < 0)
    return MC_EINVAL;
  if (!valid_dtype(w_dtype)) return MC_EDTYPE;
  if (!(tau > 0.0f) || !isfinite(tau) || !(alpha >= 0.0f && alpha <= 1.0f)) return MC_EINVAL;
  // bounds under which every element count and offset below and in the
  // kernels fits in int64 (H (qph + kph) d_in < 2^58)
  if (q_rows_per_head > 65536 || k_rows_per_head > 65536 || d_in > (int64_t{1} << 24)) return MC_ESHAPE;
  return MC_OK;
}

static mc_status_t qk_clip_common(const float* smax, int64_t H, bool total_clip, float tau, float alpha,
                                  void* Wq, void* Wk, int w_dtype, int64_t d_in, int64_t q_rows_per_head,
                                  int64_t q_c_rows, int64_t k_rows_per_head, float* gamma_out,
                                  int32_t* clipped_out, void* stream) {
  mc_status_t st = qk_clip_check(H, tau, alpha, w_dtype, d_in, q_rows_per_head, q_c_rows, k_rows_per_head);
  if (st != MC_OK) return st;
  if (H == 0) return MC_OK;
  if (!smax) return MC_EINVAL;
  if ((q_rows_per_head > 0 && !Wq) || (k_rows_per_head > 0 && !Wk)) return MC_EINVAL;
  if (H > 65535) return MC_ESHAPE;
  const size_t es = dtype_size(w_dtype);
  if (!aligned(smax, 4) || (Wq && !aligned(Wq, es)) || (Wk && !aligned(Wk, es)) ||
      (gamma_out && !aligned(gamma_out, 4)) || (clipped_out && !aligned(clipped_out, 4)))
    return MC_EALIGN;
  if ((q_rows_per_head + k_rows_per_head) * d_in / 8 / 1024 + 1 > kGridMax) return MC_ESHAPE;
  return done(mc::launch_qk_clip(smax, 1, H, total_clip, tau, alpha, &Wq, &Wk, w_dtype == MC_BF16, d_in,
                                 q_rows_per_head, q_c_rows, k_rows_per_head, gamma_out, clipped_out,
                                 static_cast<hipStream_t>(stream)),
              stream, "qk_clip_apply");
}

mc_status_t qk_clip_apply_layers(const float* smax, int64_t L, int64_t H, float tau, float alpha, void* const* Wq,
                                 void* const* Wk, int w_dtype, int64_t d_in, int64_t q_rows_per_head,
                                 int64_t q_c_rows, int64_t k_rows_per_head, float* gamma_out, int32_t* clipped_out,
                                 void* stream) {
  if (L < 0) return MC_EINVAL;
  mc_status_t st = qk_clip_check(H, tau, alpha, w_dtype, d_in, q_rows_per_head, q_c_rows, k_rows_per_head);
  if (st != MC_OK) return st;
  if (L == 0 || H == 0) return MC_OK;
  if (!smax || !Wq || !Wk) return MC_EINVAL;
  const size_t es = dtype_size(w_dtype);
  for (int64_t l = 0; l < L; ++l) {
    if ((q_rows_per_head > 0 && !Wq[l]) || (k_rows_per_head > 0 && !Wk[l])) return MC_EINVAL;
    if ((Wq[l] && !aligned(Wq[l], es)) || (Wk[l] && !aligned(Wk[l], es))) return MC_EALIGN;
  }
  if (L * H > 65535) return MC_ESHAPE;
  if (!aligned(smax, 4) || (gamma_out && !aligned(gamma_out, 4)) || (clipped_out && !aligned(clipped_out, 4)))
    return MC_EALIGN;
  if ((q_rows_per_head + k_rows_per_head) * d_in / 8 / 1024 + 1 > kGridMax) return MC_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t l0 = 0; l0 < L; l0 += mc::kClipMaxLayers) {
    const int64_t nl = L - l0 < mc::kClipMaxLayers ? L - l0 : mc::kClipMaxLayers;
    const hipError_t e = mc::launch_qk_clip(smax + l0 * H, nl, H, false, tau, alpha, Wq + l0, Wk + l0,
                                            w_dtype == MC_BF16, d_in, q_rows_per_head, q_c_rows, k_rows_per_head,
                                            gamma_out ? gamma_out + l0 * H : nullptr,
                                            clipped_out ? clipped_out + l0 * H : nullptr, s);
    if (e != hipSuccess) return MC_EHIP;
  }
  return done(hipSuccess, stream, __func__);
}

mc_status_t qk_clip_apply(const float* smax, int64_t H, float tau, float alpha, void* Wq, void* Wk,
                          int w_dtype, int64_t d_in, int64_t q_rows_per_head, int64_t q_c_rows,
                          int64_t k_rows_per_head, float* gamma_out, int32_t* clipped_out,
                          void* stream) {
  return qk_clip_common(smax, H, false, tau, alpha, Wq, Wk, w_dtype, d_in, q_rows_per_head, q_c_rows,
                        k_rows_per_head, gamma_out, clipped_out, stream);
}

mc_status_t qk_clip_apply_total(const float* smax, int64_t H, float tau, float alpha, void* Wq, void* Wk,
                                int w_dtype, int64_t d_in, int64_t q_rows_per_head, int64_t q_c_rows,
                                int64_t k_rows_per_head, float* gamma_out, int32_t* clipped_out,
                                void* stream) {
  return qk_clip_common(smax, H, true, tau, alpha, Wq, Wk, w_dtype, d_in, q_rows_per_head, q_c_rows,
                        k_rows_per_head, gamma_out, clipped_out, stream);
}

}  // extern "C"

extern "C" {

mc_status_t mc_probe_mfma_bf16(int64_t workgroups, int64_t iters, int zero_operands, float* out, void* stream) {
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (int64_t{1} << 30)) return MC_EINVAL;
  if (!out || !aligned(out, 4)) return MC_EINVAL;
  return from_hip(mc::launch_mfma_probe(workgroups, iters, zero_operands != 0, out, static_cast<hipStream_t>(stream)));
}

mc_status_t mc_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return MC_EINVAL;
  if (bytes == 0) return MC_OK;
  if (!src || !dst) return MC_EINVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MC_EALIGN;
  return from_hip(mc::launch_copy_probe(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
