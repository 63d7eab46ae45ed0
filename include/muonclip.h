/*
 * muonclip.h - C ABI of libmuonclip.so, the MuonClip optimizer step on AMD
 * Instinct MI355X (gfx950).
 *
 * The step (Algorithm 1 of "Kimi K2 内部机制", the Kimi K2 internals deep
 * dive, MuonClip section; the muonclip_step pseudocode of "Kimi K2: Open
 * Agentic Intelligence", paper notes section 3.2) is split into the calls
 * below.  A training loop calls, per step:
 *
 *   muonclip_momentum              M <- mu M + G              (every matrix)
 *   muon_ns_orthogonalize_batched  O <- NewtonSchulz(M) * s   (per shape group)
 *   muon_apply_update              W <- W - eta (O + lambda W)
 *   qk_maxlogit                    S_max^h from the forward's Q, K
 *   qk_clip_apply                  rescale W_q / W_k rows of heads over tau
 *
 * or, where the forward itself runs here, S_max comes out of the attention
 * forward (attention_fwd_maxlogit) instead of a separate qk_maxlogit pass.
 *
 * or, for the Muon part, one fused call per shape group that does the first
 * three without storing O:
 *
 *   muon_momentum_ns_update_batched  M <- mu M + G; W <- W - eta (s NS(M) + lambda W)
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller, except
 *    `coeffs` of the Newton-Schulz calls, which is host memory.  The
 *    library never allocates device memory; scratch space is a caller
 *    workspace whose size a query function returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls enqueue work on it and return without synchronising.
 *  - Argument errors are reported before anything is enqueued, and then no
 *    output is touched.  A failed launch returns MC_EHIP; the stream's work
 *    is then undefined.  No C++ exception crosses the ABI.
 *  - Apart from the allocation-free entry point's static scratch (see
 *    there) and a debug build's check flags, the library holds no mutable
 *    global state: calls on different streams may run concurrently as long
 *    as their buffers do not overlap.
 *  - Debug builds (libmuonclip_debug.so, compiled with MC_DEBUG; host code
 *    under UndefinedBehaviorSanitizer) check the index ranges of the
 *    kernels' global accesses and skip any access that fails, synchronise
 *    the stream at the end of every call and then return MC_ECHECK (with
 *    the failed checks printed to stderr) if a check failed.  Their results
 *    otherwise equal the release build's; they are for tests, not speed,
 *    and do not support overlapping calls.
 *  - Element counts and strides are in elements, not bytes.  Pointers must be
 *    aligned to their element size; wider alignment enables vector paths.
 *  - Dtypes: MC_F32 = IEEE binary32, MC_BF16 = bfloat16 (top half of binary32).
 *    Rounding to bf16 is round-to-nearest-even.
 */
#ifndef MUONCLIP_H
#define MUONCLIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MC_ABI_VERSION 2

/* Entry points are the only symbols the library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define MC_API __attribute__((visibility("default")))
#else
#define MC_API
#endif

typedef enum mc_status {
  MC_OK = 0,
  MC_EINVAL = 1,     /* null pointer, negative size, bad scalar (NaN lr, steps <= 0 ...) */
  MC_ESHAPE = 2,     /* shape outside what the call supports */
  MC_EDTYPE = 3,     /* dtype code not supported by the call */
  MC_EALIGN = 4,     /* pointer not aligned to its element size */
  MC_EWORKSPACE = 5, /* workspace missing or smaller than the query function's size */
  MC_EHIP = 6,       /* a HIP runtime call or kernel launch failed */
  MC_ECHECK = 7      /* debug builds only: a kernel's range check failed (outputs undefined) */
} mc_status_t;

typedef enum mc_dtype { MC_F32 = 0, MC_BF16 = 1 } mc_dtype_t;

/* MC_ABI_VERSION of the loaded library. */
MC_API int mc_abi_version(void);

/* 1 for a debug build (MC_DEBUG range checks, see above), else 0. */
MC_API int mc_debug_build(void);

/* Static, human-readable name of a status code (never NULL). */
MC_API const char* mc_status_string(int status);

/*
 * Momentum accumulation: M <- fl32(fl32(mu * M) + G), element-wise, in place.
 *
 * Defined by Algorithm 1 of the internals deep dive (M_t = mu M_{t-1} + G_t,
 * M_0 = 0) and the paper-notes pseudocode, which performs it as a scale of M
 * followed by an add of G: two float32 roundings, never a fused multiply-add,
 * so the result is bit-identical to float32 multiply-then-add.
 *
 *   M      device float32[numel], read and written
 *   G      device float32[numel], read
 *   numel  >= 0 (0 enqueues nothing); several matrices may be passed as one
 *          flat concatenated buffer, since the op is element-wise
 *   mu     momentum (0.95 on the pages), used as given in float32
 * Errors: MC_EINVAL (null pointer with numel > 0, numel < 0), MC_EALIGN.
 */
MC_API mc_status_t muonclip_momentum(float* M, const float* G, int64_t numel, float mu, void* stream);

/*
 * The Muon output scale sqrt(max(rows, cols)) * 0.2, which matches the RMS of
 * the update to AdamW's (Algorithm 1 of "Kimi K2 内部机制": O_t =
 * NewtonSchulz(M_t) * sqrt(max(n, m)) * 0.2; the Zhihu MuonClip formula,
 * "Match Adam Update RMS"), computed in double and rounded once to float32.
 * Returns 0 when rows < 1 or cols < 1.
 */
MC_API float muon_rms_match_scale(int64_t rows, int64_t cols);

/* Pass as out_scale to the Newton-Schulz calls to have the library apply
 * muon_rms_match_scale(rows, cols); every negative out_scale does the same. */
#define MC_OUT_SCALE_RMS_MATCH (-1.0f)

/*
 * Workspace bytes that muon_ns_orthogonalize_batched needs for `batch`
 * matrices of rows x cols.  Returns 0 for invalid or unsupported sizes
 * (those the Newton-Schulz calls reject with MC_EINVAL or MC_ESHAPE).
 */
MC_API size_t muon_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols);

/*
 * Batched Newton-Schulz orthogonalisation with the Muon output scale:
 *   O_b = out_scale * NS(M_b)      for b in [0, batch)
 * where, for one matrix M (rows x cols):
 *   X_0 = M / (||M||_F + eps), taken as its transpose when rows > cols
 *         (n = min(rows, cols) rows, m = max(rows, cols) columns);
 *   for s in [0, steps): A = X X^T; B = b_s A + c_s A A; X <- a_s X + B X;
 *   NS(M) = X (transposed back when rows > cols).
 * The pages define O_t = NewtonSchulz(M_t) * sqrt(max(n, m)) * 0.2 (Algorithm 1
 * of the internals deep dive; msign in the Zhihu thread's MuonClip formula) and
 * describe Newton-Schulz only as a few iterations of an odd polynomial driving
 * the singular values toward 1 ("Kimi K2, explained.", Muon update bullets).
 * The polynomial coefficients, the step count and the Frobenius pre-scale are
 * not on the pages and are arguments here.  Pass out_scale =
 * MC_OUT_SCALE_RMS_MATCH (any negative value) for the pages' step: the
 * library then uses muon_rms_match_scale(rows, cols).
 *
 * Arithmetic: the norm is accumulated in float32 (combined in double); X_0
 * is held unscaled and the factor 1 / (||M||_F + eps) is applied in float32
 * by the first step's GEMMs (X X^T by its square, that step's X by it).  X
 * is carried as X = Xh + Xl, a bf16 high part and the rounding residual as
 * one signed byte per element, a step of 256 in the binary32 bit pattern
 * from the high part's (about 16 significant bits together); each step computes A = Xh Xh^T and B = b_s A + c_s A A on bf16 MFMA
 * with float32 accumulation (A rounded to bf16; B's diagonal d kept in
 * float32 and the rest rounded to bf16), then X <- a_s X + d Xh + N Xh (N =
 * B off its diagonal) in float32, split into its two parts again.  Keeping
 * a_s X exact to 16 bits stops rounding errors from growing along the small
 * singular directions (where a step multiplies by about a_s), so low-rank
 * and decaying spectra keep the Gaussian case's accuracy.  The last step's
 * X is rounded to bf16 before out_scale is applied.
 *
 *   M              device, m_dtype (MC_F32 or MC_BF16); matrix b starts at
 *                  element b * m_batch_stride and is row-major rows x cols
 *   O              device, o_dtype, same layout with o_batch_stride; O may be
 *                  the same buffer as M when dtypes and strides match
 *   steps          1..64; coeffs: host float[steps][3] = (a_s, b_s, c_s)
 *   eps            >= 0; out_scale: finite; negative = the RMS-matching
 *                  scale sqrt(max(rows, cols)) * 0.2
 *   workspace      device, >= muon_ns_workspace_bytes(batch, rows, cols)
 *                  bytes, 256-byte aligned; contents on entry are ignored
 *   gemm_events    NULL, or host array of 6 * steps hipEvent_t (as void*):
 *                  events[2*(3s+g)] and events[2*(3s+g)+1] are recorded on
 *                  `stream` right before and after GEMM g of step s
 *                  (g = 0: X X^T, 1: b A + c A A, 2: a X + B X), for timing
 * Sizes: batch >= 0 (0 enqueues nothing); 1 <= rows, cols; min(rows, cols)
 * <= 16384 and max(rows, cols) <= 65536; batch <= 65535 and batch times the
 * number of 256 x 256 tiles of X below 2^31 (else MC_ESHAPE).
 * Errors: MC_EINVAL, MC_ESHAPE, MC_EDTYPE, MC_EALIGN, MC_EWORKSPACE, MC_EHIP.
 */
MC_API mc_status_t muon_ns_orthogonalize_batched(const void* M, int m_dtype, int64_t batch, int64_t rows,
                                          int64_t cols, int64_t m_batch_stride, void* O, int o_dtype,
                                          int64_t o_batch_stride, int32_t steps, const float* coeffs,
                                          float eps, float out_scale, void* workspace,
                                          size_t workspace_bytes, void* stream,
                                          void* const* gemm_events);

/*
 * Decoupled weight-decay update: W <- W - lr * (O + weight_decay * W),
 * element-wise, in place (Algorithm 1 of the internals deep dive; the
 * paper-notes pseudocode W.add_(O + weight_decay * W, alpha=-lr)).
 * Computed in float32 as t = weight_decay * W; u = O + t; v = lr * u;
 * W' = W - v (no fused multiply-add), rounded once to W's dtype.
 *
 *   W      device, w_dtype (MC_F32 or MC_BF16), numel elements
 *   O      device, o_dtype (MC_F32 or MC_BF16), numel elements, same layout
 *   numel  >= 0; lr, weight_decay finite
 * Errors: MC_EINVAL, MC_EDTYPE, MC_EALIGN, MC_EHIP.
 */
MC_API mc_status_t muon_apply_update(void* W, int w_dtype, const void* O, int o_dtype, int64_t numel,
                              float lr, float weight_decay, void* stream);

/*
 * The Muon part of the step for a batch of equally shaped matrices, fused:
 * for b in [0, batch), with M_b, G_b, W_b rows x cols at element offset
 * b * batch_stride of M, G and W,
 *   M_b <- fl32(fl32(mu * M_b) + G_b)                      (as muonclip_momentum)
 *   O_b  = out_scale * NS(M_b)                             (as muon_ns_orthogonalize_batched)
 *   W_b <- W_b - lr * (O_b + weight_decay * W_b)           (as muon_apply_update)
 * (Algorithm 1 of "Kimi K2 内部机制", MuonClip section; the paper notes'
 * muonclip_step pseudocode, section 3.2.)  The momentum is bit-identical to
 * muonclip_momentum.  O is never stored: the last Newton-Schulz GEMM applies
 * the update as it finishes each tile of X (X rounded to bf16 as in the
 * output of muon_ns_orthogonalize_batched; O = out_scale * X formed in
 * float32, not rounded to a storage type).  The new M is converted to its
 * (bf16, int8 code) pair once, in the momentum pass, together with float32 partial sums
 * of its squares; the normalisation
 * 1 / (||M_b||_F + eps) is applied inside the first Newton-Schulz step (to
 * X X^T squared and to the step's result), which equals normalising X_0 up
 * to rounding.  Steps and coefficients as muon_ns_orthogonalize_batched.
 *
 *   M          device float32, in/out;  G: device float32
 *   W          device, w_dtype (MC_F32 or MC_BF16), in/out
 *   batch_stride  elements between consecutive matrices of M, G and W
 *                 (>= rows * cols when batch > 1)
 *   mu, lr, weight_decay, out_scale: finite; eps >= 0; out_scale < 0
 *                 (MC_OUT_SCALE_RMS_MATCH) = sqrt(max(rows, cols)) * 0.2, the
 *                 pages' step
 *   workspace  device, >= muon_ns_workspace_bytes(batch, rows, cols) bytes,
 *              256-byte aligned
 *   gemm_events as muon_ns_orthogonalize_batched (the last step's third GEMM
 *              includes the update)
 * Sizes as muon_ns_orthogonalize_batched.
 * Errors: MC_EINVAL, MC_ESHAPE, MC_EDTYPE, MC_EALIGN, MC_EWORKSPACE, MC_EHIP.
 */
MC_API mc_status_t muon_momentum_ns_update_batched(float* M, const float* G, float mu, void* W, int w_dtype,
                                                   int64_t batch, int64_t rows, int64_t cols,
                                                   int64_t batch_stride, int32_t steps, const float* coeffs,
                                                   float eps, float out_scale, float lr, float weight_decay,
                                                   void* workspace, size_t workspace_bytes, void* stream,
                                                   void* const* gemm_events);

/*
 * muon_momentum_ns_update_batched_noalloc -- the same fused Muon call for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace: its scratch is a static device array of the library,
 * MC_NOALLOC_SCRATCH_BYTES (192 MiB) on each GPU the library runs on, held
 * from the library's first use on that GPU until the process ends.  The
 * call itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller passes M, G, W and the coefficients as for
 * muon_momentum_ns_update_batched, with the same results bit for bit.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (no part of it needs to start at zero: each call writes
 * every byte it reads).  Calls that overlap in time on one GPU (different
 * streams, or host threads) race on it and give undefined results: order
 * them on one stream.  The GPU of a call is the device of its stream (the
 * calling thread's current device for the null stream); M, G and W must be
 * on it.  The first call on a GPU looks up the array's address
 * (hipGetSymbolAddress) with that GPU made current, then restores the
 * thread's current device; later calls reuse the address.
 *
 * Arguments, sizes and errors as muon_momentum_ns_update_batched, plus
 * MC_EWORKSPACE when muon_ns_workspace_bytes(batch, rows, cols) exceeds
 * MC_NOALLOC_SCRATCH_BYTES (for example one 2048 x 7168 matrix fits, a
 * batch of two does not), and MC_EHIP when the address lookup fails.
 */
#define MC_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
MC_API mc_status_t muon_momentum_ns_update_batched_noalloc(float* M, const float* G, float mu, void* W,
                                                           int w_dtype, int64_t batch, int64_t rows, int64_t cols,
                                                           int64_t batch_stride, int32_t steps,
                                                           const float* coeffs, float eps, float out_scale,
                                                           float lr, float weight_decay, void* stream);

/*
 * Per-head max logit over a batch, the logits never stored:
 *   S_max^h = (1/sqrt(d)) * max_{b, i, j} Q[b,h,i,:] . K[b,h,j,:]
 * with K[b,h,j,:] = [Kc[b,h,j,0:d_c] || Kr[b,j,0:d_r]] (MLA: the rotary key
 * part is shared by all heads) or Kc alone when d_r = 0 (MHA), d = d_c + d_r.
 * Defined in "Kimi K2 内部机制", MuonClip section, core maths (max over the
 * batch and over all token pairs of the scaled dot product); the paper notes
 * print 1/d, read as 1/sqrt(d).  No causal mask: every (i, j) pair counts.
 * Logits that are NaN are skipped; a head with no numeric logit gets -inf.
 *
 *   Q      device [B, H, Sq, d] row-major, dtype
 *   Kc     device [B, H, Sk, d_c] row-major, dtype
 *   Kr     device [B, Sk, d_r] row-major, dtype; NULL iff d_r == 0
 *   dtype  MC_BF16 (bf16 MFMA, float32 accumulation) or MC_F32 (float32 FMA)
 *   smax   device float32[H]: overwritten when accumulate == 0; when
 *          accumulate != 0 the result is max(smax, S_max) (batches split over
 *          several calls)
 * Sizes: B, H, Sq, Sk >= 1 (any zero enqueues nothing but the overwrite of
 * smax with -inf); 1 <= d_c; 0 <= d_r; d <= 512.
 * Errors: MC_EINVAL, MC_ESHAPE, MC_EDTYPE, MC_EALIGN, MC_EHIP.
 */
MC_API mc_status_t qk_maxlogit(const void* Q, const void* Kc, const void* Kr, int dtype, int64_t B, int64_t H,
                        int64_t Sq, int64_t Sk, int64_t d_c, int64_t d_r, float* smax,
                        int32_t accumulate, void* stream);

/*
 * attention_fwd_maxlogit -- attention forward with the per-head max logit as
 * a by-product (the logits are never written anywhere):
 *   O[b,h,i,:] = sum_j softmax_j(L[b,h,i,j]) V[b,h,j,:],
 *   L[b,h,i,j] = Q[b,h,i,:] . K[b,h,j,:] / sqrt(d_c + d_r),
 *   smax[h]    = max over b, i and visible j of L[b,h,i,j],
 *   lse[b,h,i] = log sum_j exp(L[b,h,i,j])   (natural log),
 * K as in qk_maxlogit (MLA: [Kc || shared Kr]; MHA: Kr = NULL, d_r = 0).
 * causal != 0: query i sees key j only when j <= i + Sk - Sq (the queries are
 * the last Sq positions; requires Sq <= Sk); hidden keys are left out of the
 * softmax and of the max.  Defined in "Kimi K2 内部机制", MuonClip section
 * (S_max is already computed in the forward) and the attention formula of
 * the paper notes ("Kimi K2: Open Agentic Intelligence", section 3.2).
 *
 *   Q   [B, H, Sq, d_c + d_r]   Kc [B, H, Sk, d_c]   Kr [B, Sk, d_r] or NULL
 *   V   [B, H, Sk, d_v]         O  [B, H, Sq, d_v]  (all bf16, row-major, device)
 *   lse_out   device float32 [B, H, Sq] or NULL
 *   smax_out  device float32 [H]; initialised to -inf first unless
 *             accumulate != 0 (then maxed into, for a batch split over calls)
 * O is computed in float32 (softmax weights rounded to bf16 for the second
 * product) and rounded once to bf16.
 * Supported: dtype MC_BF16 (else MC_EDTYPE); (d_c, d_r, d_v) = (128, 64, 128)
 * (Kimi K2's MLA head) or (64, 0, 64) (else MC_ESHAPE); Sk >= 64 unless the
 * call is empty (B, H or Sq zero: then only smax_out is written, -inf unless
 * accumulating, and the other pointers may be NULL); Q, Kc, Kr, V 16-byte
 * aligned, O 8-byte aligned (MC_EALIGN).
 * Errors: MC_EINVAL, MC_ESHAPE, MC_EDTYPE, MC_EALIGN, MC_EHIP.
 */
MC_API mc_status_t attention_fwd_maxlogit(const void* Q, const void* Kc, const void* Kr, const void* V,
                                          int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t d_c,
                                          int64_t d_r, int64_t d_v, int32_t causal, void* O, float* lse_out,
                                          float* smax_out, int32_t accumulate, void* stream);

/*
 * QK-Clip: for each head h with smax[h] > tau, gamma = tau / smax[h] and
 *   W_q rows [h*qph, h*qph + q_c_rows)      *= gamma^alpha
 *   W_q rows [h*qph + q_c_rows, (h+1)*qph)  *= gamma
 *   W_k rows [h*kph, (h+1)*kph)             *= gamma^(1 - alpha)
 * (qph = q_rows_per_head, kph = k_rows_per_head), in place, computed in
 * float32 and rounded once to w_dtype.  Heads with smax[h] <= tau or NaN are
 * not touched (bit-for-bit).  MLA: q_c_rows = nope rows, the rest of the head
 * is the head-specific rotary query q^R, W_k is W_kc, and the shared rotary
 * key is simply not passed; MHA: q_c_rows = q_rows_per_head.
 * Defined in "Kimi K2 内部机制", MuonClip section: gamma_h = min(1, tau/S_max^h),
 * only heads over tau touched, W_q^h by gamma^alpha and W_k^h by
 * gamma^(1-alpha), and the MLA table (q^C, k^C by sqrt(gamma); q^R by gamma;
 * shared k^R untouched); the paper-notes pseudocode skips heads at or below
 * tau.  gamma^0.5 uses a correctly rounded sqrt, other exponents powf.
 *
 *   smax         device float32[H]
 *   Wq, Wk       device, w_dtype, row-major [H*qph, d_in] and [H*kph, d_in]
 *   gamma_out    device float32[H] or NULL: gamma (1 for untouched heads)
 *   clipped_out  device int32[H] or NULL: 1 clipped, 0 not, -1 smax was NaN
 * Sizes: H >= 0; d_in >= 1; 0 <= q_c_rows <= qph; kph >= 0; H <= 65535,
 * qph, kph <= 65536 and d_in <= 2^24 (else MC_ESHAPE).
 * Errors: MC_EINVAL (also tau not finite and > 0, alpha outside [0, 1]),
 * MC_ESHAPE, MC_EDTYPE, MC_EALIGN, MC_EHIP.
 */
MC_API mc_status_t qk_clip_apply(const float* smax, int64_t H, float tau, float alpha, void* Wq, void* Wk,
                          int w_dtype, int64_t d_in, int64_t q_rows_per_head, int64_t q_c_rows,
                          int64_t k_rows_per_head, float* gamma_out, int32_t* clipped_out,
                          void* stream);

/*
 * qk_clip_apply_layers -- QK-Clip of every attention layer in one call: for
 * each layer l and head h with smax[l * H + h] > tau, the rows of head h of
 * layer l's W_q and W_k are rescaled exactly as qk_clip_apply rescales them
 * (the pages clip every head of every attention layer: Algorithm 1 of "Kimi
 * K2 内部机制" loops over the heads of each attention layer; the Zhihu
 * MuonClip formula indexes S_max by layer and head).
 *
 *   smax         device float32 [L, H] row-major (the forward's per-layer
 *                per-head max logits)
 *   Wq, Wk       HOST arrays of L device pointers: layer l's W_q
 *                [H*qph, d_in] and W_k [H*kph, d_in] (same dtype, shapes and
 *                row split for every layer)
 *   gamma_out    device float32 [L, H] or NULL;  clipped_out device int32
 *                [L, H] or NULL (1 clipped, 0 not, -1 NaN)
 * Up to 64 layers go in one kernel launch (their pointers travel in the
 * kernel arguments); more layers take one launch per 64.  Arguments and
 * errors otherwise as qk_clip_apply, plus MC_EINVAL for L < 0, a NULL
 * pointer array or a NULL layer pointer, and MC_ESHAPE for L * H > 65535.
 */
MC_API mc_status_t qk_clip_apply_layers(const float* smax, int64_t L, int64_t H, float tau, float alpha,
                                        void* const* Wq, void* const* Wk, int w_dtype, int64_t d_in,
                                        int64_t q_rows_per_head, int64_t q_c_rows, int64_t k_rows_per_head,
                                        float* gamma_out, int32_t* clipped_out, void* stream);

/*
 * qk_clip_apply_total -- the total-clip variant: one gamma for all heads.
 *
 * S = max_h smax[h] (NaN entries skipped); if S > tau, gamma = tau / S and
 * every head's rows are rescaled exactly as qk_clip_apply rescales a clipped
 * head (q_c_rows x gamma^alpha, the rest of the head's W_q rows x gamma, W_k
 * rows x gamma^(1-alpha)); otherwise nothing is touched.  Defined in
 * "Kimi K2 内部机制", MuonClip section: the naive form that clips all heads
 * together with gamma = min(1, tau / S_max), S_max = max_h S_max^h, before
 * the per-head gamma_h replaces it (the Zhihu answer also names the change
 * from total clip to per-head clip).  gamma_out / clipped_out get the same
 * value for every head (clipped 1 or 0; -1 when every smax is NaN).
 * Arguments, layouts and errors as for qk_clip_apply.
 */
MC_API mc_status_t qk_clip_apply_total(const float* smax, int64_t H, float tau, float alpha, void* Wq,
                                       void* Wk, int w_dtype, int64_t d_in, int64_t q_rows_per_head,
                                       int64_t q_c_rows, int64_t k_rows_per_head, float* gamma_out,
                                       int32_t* clipped_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUONCLIP_H */
