// Host-side launch interface of the libwandit kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.hpp"

namespace wan {

enum OutKind { OUT_BF16 = 0, OUT_F32 = 1, OUT_GELU = 2, OUT_RESID = 3 };

// C[M,N] = A[M,K] . B[N,K]^T (+ bias) with an epilogue.
struct GemmDesc {
  const void *A; long lda;     // [M, K]
  const void *B; long ldb;     // [N, K]
  int M, N, K;
  const void *bias;            // [N] (or [M] when bias_rows), may be NULL
  int bias_rows;
  int kind;                    // OutKind
  void *C; long ldc;           // OUT_BF16 / OUT_F32 / OUT_GELU destination
  // OUT_RESID: x[m, n] += gate[b(m), n] * (acc + bias[n]); gate may be NULL (=1)
  float *X; long ldx;
  const float *gate; long gate_bstride; int rows_per_batch;
  int f32;                     // operands / bias / C are float32 instead of bf16
  int npad;                    // OUT_BF16: columns N .. npad-1 of C are written as zeros
  // FP8 (OCP E4M3) operands: A and B hold one byte per element, K % 64 == 0;
  // acc is multiplied by a_scale[a_per_row ? m : 0] * b_scale[b_per_col ? n : 0]
  // before the bias (per-token / per-tensor dequantisation, either side)
  int fp8;
  const float *a_scale, *b_scale;
  int a_per_row, b_per_col;
  // OUT_BF16: columns 0 .. scale_cols-1 (a multiple of 8) are multiplied by
  // col_scale after the bias, before the rounding (attention's pre-scaled Q)
  int scale_cols;
  float col_scale;
};


hipError_t launch_mod_combine(const float *mod, const float *bias, float *out, int B, int n,
                              hipStream_t s);
hipError_t launch_ln_mod(const float *x, int M, int L, int d, const float *modb, long modb_bstride,
                         int shift_off, int scale_off, int has_mod, float eps, void *out,
                         int out_f32, hipStream_t s);
// LayerNorm (+ modulate) straight to E4M3 codes and per-row scales (widths
// for which ln_mod_fp8_supported holds)
hipError_t launch_ln_mod_fp8(const float *x, int M, int L, int d, const float *modb,
                             long modb_bstride, int shift_off, int scale_off, int has_mod, float eps,
                             void *q, float *scale, hipStream_t s);
bool ln_mod_fp8_supported(int d);
hipError_t launch_gemm(const GemmDesc &g, hipStream_t s);
hipError_t launch_tmlp(const float *t, int B, int freq_dim, int d, const void *w1, const void *b1,
                       const void *w2, const void *b2, float *hidden, float *mod, int f32,
                       hipStream_t s);
hipError_t launch_patch_gather(const float *latent, int B, int C, int F, int H8, int W8, int Kp,
                               void *P, int f32, hipStream_t s);
hipError_t launch_head_unpatchify(const float *x, int B, int F, int Hp, int Wp, int d,
                                  const void *w, const void *b, int out_ch, float *out, int f32,
                                  hipStream_t s);
hipError_t launch_pad_rows(const void *src, int R, int K, int Kp, void *dst, int f32, hipStream_t s);
hipError_t launch_fill(float *p, int n, float v, hipStream_t s);
// FP8 (OCP E4M3) quantisation: per row (one scale per row) and per tensor
hipError_t launch_quant_rows_fp8(const void *x, int M, int K, long ldx, void *q, long ldq,
                                 float *scale, hipStream_t s);
hipError_t launch_quant_tensor_fp8(const void *w, long n, void *q, float *scale, unsigned *amax_bits,
                                   hipStream_t s);
hipError_t launch_euler(float *lat, const float *vel, int B, int in_ch, int out_ch, long plane,
                        float dt, int guided, float scale, hipStream_t s);

}  // namespace wan
