/*
 * A plain C client of libmuonclip.so: one MuonClip step through the C ABI
 * alone (HIP runtime for device memory and a stream; no Python, no torch).
 *
 *   step_client IN OUT
 *
 * IN (little-endian): 13 int64 -- batch, rows, cols of the Muon matrices;
 * B, H, Sq, Sk, d_c, d_r of the forward's Q [B,H,Sq,d_c+d_r], Kc [B,H,Sk,d_c],
 * Kr [B,Sk,d_r]; q_rows_per_head, q_c_rows, k_rows_per_head, d_in of W_q
 * [H*q_rows_per_head, d_in] and W_k [H*k_rows_per_head, d_in] -- then float32
 * M, G, W (batch x rows x cols each), bf16 bit patterns of Q, Kc, Kr, and
 * float32 W_q, W_k.
 *
 * The step ("Kimi K2 内部机制", MuonClip, Algorithm 1): the fused Muon call
 * (M <- 0.95 M + G; W <- W - 2e-3 (0.2 sqrt(max(rows, cols)) NS5(M) + 0.1 W),
 * the public Muon quintic), the per-head max logit of Q, K, and QK-Clip of
 * W_q, W_k at tau 100, alpha 0.5.
 *
 * OUT: float32 M, W, S_max [H], gamma [H], int32 clipped [H], float32 W_q, W_k.
 * Exit status 0 on success; 1 usage or file errors, 2 HIP errors, 3 library
 * errors (the status string is printed).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "muonclip.h"

#define HIP_OK(x)                                                           \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define MC_OK_(x)                                                           \
  do {                                                                      \
    mc_status_t s_ = (x);                                                   \
    if (s_ != MC_OK) {                                                      \
      fprintf(stderr, "%s: %s\n", #x, mc_status_string(s_));                \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static int fail(const char* what) {
  fprintf(stderr, "step_client: %s\n", what);
  return 1;
}

enum { N_IN = 8, N_DEV = 12 };  /* the first N_IN buffers are read from IN */

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("cannot open the input file");
  int64_t h[13];
  if (fread(h, sizeof h, 1, in) != 1) return fail("short input header");
  const int64_t batch = h[0], rows = h[1], cols = h[2], B = h[3], H = h[4], Sq = h[5], Sk = h[6], d_c = h[7],
                d_r = h[8], qph = h[9], q_c_rows = h[10], kph = h[11], d_in = h[12];
  const int64_t nw = batch * rows * cols;
  /* host and device buffers: M, G, W, Q, Kc, Kr, Wq, Wk (inputs), smax, gamma, clipped, workspace */
  const size_t bytes[N_DEV] = {
      (size_t)nw * 4, (size_t)nw * 4, (size_t)nw * 4,
      (size_t)(B * H * Sq * (d_c + d_r)) * 2, (size_t)(B * H * Sk * d_c) * 2, (size_t)(B * Sk * d_r) * 2,
      (size_t)(H * qph * d_in) * 4, (size_t)(H * kph * d_in) * 4,
      (size_t)H * 4, (size_t)H * 4, (size_t)H * 4, muon_ns_workspace_bytes(batch, rows, cols)};
  void* host[N_DEV] = {0};
  void* dev[N_DEV] = {0};
  for (int i = 0; i < N_DEV; ++i) {
    host[i] = malloc(bytes[i] ? bytes[i] : 1);
    if (!host[i]) return fail("out of host memory");
    if (bytes[i]) HIP_OK(hipMalloc(&dev[i], bytes[i]));
  }
  for (int i = 0; i < N_IN; ++i)
    if (bytes[i] && fread(host[i], bytes[i], 1, in) != 1) return fail("short input file");
  fclose(in);
  for (int i = 0; i < N_IN; ++i)
    if (bytes[i]) HIP_OK(hipMemcpy(dev[i], host[i], bytes[i], hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  float coeffs[15];
  for (int s = 0; s < 5; ++s) {
    coeffs[3 * s] = 3.4445f;
    coeffs[3 * s + 1] = -4.7750f;
    coeffs[3 * s + 2] = 2.0315f;
  }
  MC_OK_(muon_momentum_ns_update_batched((float*)dev[0], (const float*)dev[1], 0.95f, dev[2], MC_F32, batch, rows,
                                         cols, rows * cols, 5, coeffs, 1e-7f, MC_OUT_SCALE_RMS_MATCH, 2e-3f, 0.1f,
                                         dev[11], bytes[11], stream, NULL));
  MC_OK_(qk_maxlogit(dev[3], dev[4], d_r > 0 ? dev[5] : NULL, MC_BF16, B, H, Sq, Sk, d_c, d_r, (float*)dev[8], 0,
                     stream));
  MC_OK_(qk_clip_apply((const float*)dev[8], H, 100.0f, 0.5f, dev[6], dev[7], MC_F32, d_in, qph, q_c_rows, kph,
                       (float*)dev[9], (int32_t*)dev[10], stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipStreamDestroy(stream));

  FILE* out = fopen(argv[2], "wb");
  if (!out) return fail("cannot open the output file");
  const int order[7] = {0, 2, 8, 9, 10, 6, 7};  /* M, W, S_max, gamma, clipped, W_q, W_k */
  for (int k = 0; k < 7; ++k) {
    const int i = order[k];
    if (!bytes[i]) continue;
    HIP_OK(hipMemcpy(host[i], dev[i], bytes[i], hipMemcpyDeviceToHost));
    if (fwrite(host[i], bytes[i], 1, out) != 1) return fail("cannot write the output file");
  }
  fclose(out);
  for (int i = 0; i < N_DEV; ++i) {
    if (dev[i]) HIP_OK(hipFree(dev[i]));
    free(host[i]);
  }
  return 0;
}
