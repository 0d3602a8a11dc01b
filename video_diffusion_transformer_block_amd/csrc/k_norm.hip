// LayerNorm (+ AdaLN modulation) over the model width, float32 residual in,
// bf16 (or float32) out.  Bandwidth-bound: 4 B read + 2 B written per
// element.  One 64-wide wavefront owns one token row; the row stays in
// registers between the mean and the variance pass.
//
// The operation: x^ = (x - mean) / sqrt(var + eps) with the biased variance
// and no affine parameters, then h = x^ (1 + scale) + shift, where shift and
// scale come from the shared timestep MLP plus the block's own bias
// ("Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)",
// section Diffusion Transformer: shared AdaLN, per-block biases).
#include "common.hpp"
#include "fp8.hpp"
#include "kernels.hpp"

namespace wan {

// modb[b, j] = mod[b, j] + bias[j]   (per block: shared MLP output + own bias)
__global__ void k_mod_combine(const float *__restrict__ mod, const float *__restrict__ bias,
                              float *__restrict__ out, int B, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * n) return;
  out[i] = mod[i] + bias[i % n];
}

template <typename OutT> WAN_DEV void store4(OutT *p, float a, float b, float c, float d);
template <> WAN_DEV void store4<bf16>(bf16 *p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = f2bf(a); v[1] = f2bf(b); v[2] = f2bf(c); v[3] = f2bf(d);
  *reinterpret_cast<bf16x4 *>(p) = v;
}
template <> WAN_DEV void store4<float>(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Row kept in registers: d = NCH * 256 (NCH float4 per lane).
template <int NCH, typename OutT>
__global__ __launch_bounds__(256) void k_ln_mod_reg(const float *__restrict__ x, int M, int L,
                                                    const float *__restrict__ modb, long modb_bs,
                                                    int shift_off, int scale_off, int has_mod,
                                                    float eps, OutT *__restrict__ out) {
  constexpr int D = NCH * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4 *xr = reinterpret_cast<const float4 *>(x + (long)row * D);
  float4 v[NCH];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    v[c] = xr[c * 64 + lane];
    s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
  }
  const float mean = wave_sum(s) * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    float a = v[c].x - mean, b = v[c].y - mean, e = v[c].z - mean, f = v[c].w - mean;
    q += (a * a + b * b) + (e * e + f * f);
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / D) + eps);
  OutT *o = out + (long)row * D;
  if (has_mod) {
    const int b = row / L;
    const float4 *sh = reinterpret_cast<const float4 *>(modb + b * modb_bs + shift_off);
    const float4 *sc = reinterpret_cast<const float4 *>(modb + b * modb_bs + scale_off);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float4 h = sh[c * 64 + lane], k = sc[c * 64 + lane];
      store4<OutT>(o + (c * 64 + lane) * 4, (v[c].x - mean) * rstd * (1.f + k.x) + h.x,
                   (v[c].y - mean) * rstd * (1.f + k.y) + h.y,
                   (v[c].z - mean) * rstd * (1.f + k.z) + h.z,
                   (v[c].w - mean) * rstd * (1.f + k.w) + h.w);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      store4<OutT>(o + (c * 64 + lane) * 4, (v[c].x - mean) * rstd, (v[c].y - mean) * rstd,
                   (v[c].z - mean) * rstd, (v[c].w - mean) * rstd);
  }
}

// The same row in E4M3 for an FP8 GEMM: each output is rounded to bf16 (the
// activation a bf16 model holds), then the row is quantised with its own
// scale (fp8.hpp): codes q[row, :] and scale[row].  Identical to the bf16
// output followed by the per-token quantiser, without the bf16 round trip.
template <int NCH>
__global__ __launch_bounds__(256) void k_ln_mod_fp8(const float *__restrict__ x, int M, int L,
                                                    const float *__restrict__ modb, long modb_bs,
                                                    int shift_off, int scale_off, int has_mod,
                                                    float eps, uint8_t *__restrict__ q,
                                                    float *__restrict__ scale) {
  constexpr int D = NCH * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4 *xr = reinterpret_cast<const float4 *>(x + (long)row * D);
  float4 v[NCH];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    v[c] = xr[c * 64 + lane];
    s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
  }
  const float mean = wave_sum(s) * (1.0f / D);
  float qs = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    float a = v[c].x - mean, b = v[c].y - mean, e = v[c].z - mean, f = v[c].w - mean;
    qs += (a * a + b * b) + (e * e + f * f);
  }
  const float rstd = rsqrtf(wave_sum(qs) * (1.0f / D) + eps);
  const int b = row / L;
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    float4 y;
    if (has_mod) {
      const float4 h = reinterpret_cast<const float4 *>(modb + b * modb_bs + shift_off)[c * 64 + lane];
      const float4 k = reinterpret_cast<const float4 *>(modb + b * modb_bs + scale_off)[c * 64 + lane];
      y = make_float4((v[c].x - mean) * rstd * (1.f + k.x) + h.x, (v[c].y - mean) * rstd * (1.f + k.y) + h.y,
                      (v[c].z - mean) * rstd * (1.f + k.z) + h.z, (v[c].w - mean) * rstd * (1.f + k.w) + h.w);
    } else {
      y = make_float4((v[c].x - mean) * rstd, (v[c].y - mean) * rstd, (v[c].z - mean) * rstd,
                      (v[c].w - mean) * rstd);
    }
    y = make_float4(bf2f(f2bf(y.x)), bf2f(f2bf(y.y)), bf2f(f2bf(y.z)), bf2f(f2bf(y.w)));
    m = fmaxf(fmaxf(m, fmaxf(fabsf(y.x), fabsf(y.y))), fmaxf(fabsf(y.z), fabsf(y.w)));
    v[c] = y;
  }
  m = wave_max(m);
  const float inv = inv_scale(m);
  unsigned *o = reinterpret_cast<unsigned *>(q + (long)row * D);
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    o[c * 64 + lane] = pack4(v[c].x * inv, v[c].y * inv, v[c].z * inv, v[c].w * inv);
  if (lane == 0) scale[row] = deq_scale(m);
}

// Any width: three passes over the row (mean, variance, output).
template <typename OutT>
__global__ __launch_bounds__(256) void k_ln_mod_any(const float *__restrict__ x, int M, int L, int D,
                                                    const float *__restrict__ modb, long modb_bs,
                                                    int shift_off, int scale_off, int has_mod,
                                                    float eps, OutT *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float *xr = x + (long)row * D;
  float s = 0.f;
  for (int i = lane; i < D; i += 64) s += xr[i];
  const float mean = wave_sum(s) / D;
  float q = 0.f;
  for (int i = lane; i < D; i += 64) { float a = xr[i] - mean; q += a * a; }
  const float rstd = rsqrtf(wave_sum(q) / D + eps);
  const int b = row / L;
  for (int i = lane; i < D; i += 64) {
    float y = (xr[i] - mean) * rstd;
    if (has_mod) y = y * (1.f + modb[b * modb_bs + scale_off + i]) + modb[b * modb_bs + shift_off + i];
    out[(long)row * D + i] = from_f<OutT>(y);
  }
}

hipError_t launch_mod_combine(const float *mod, const float *bias, float *out, int B, int n,
                              hipStream_t s) {
  int tot = B * n;
  k_mod_combine<<<(tot + 255) / 256, 256, 0, s>>>(mod, bias, out, B, n);
  return hipGetLastError();
}

template <typename OutT>
static hipError_t ln_dispatch(const float *x, int M, int L, int d, const float *modb, long bs,
                              int so, int co, int hm, float eps, OutT *out, hipStream_t s) {
  dim3 grid((M + 3) / 4), blk(256);
#define WAN_LN_CASE(n) \
  case n: k_ln_mod_reg<n, OutT><<<grid, blk, 0, s>>>(x, M, L, modb, bs, so, co, hm, eps, out); break;
  if (d % 256 == 0 && d / 256 <= 24) {
    switch (d / 256) {
      WAN_LN_CASE(1) WAN_LN_CASE(2) WAN_LN_CASE(3) WAN_LN_CASE(4) WAN_LN_CASE(5) WAN_LN_CASE(6)
      WAN_LN_CASE(8) WAN_LN_CASE(10) WAN_LN_CASE(12) WAN_LN_CASE(16) WAN_LN_CASE(20) WAN_LN_CASE(24)
      default: k_ln_mod_any<OutT><<<grid, blk, 0, s>>>(x, M, L, d, modb, bs, so, co, hm, eps, out);
    }
  } else {
    k_ln_mod_any<OutT><<<grid, blk, 0, s>>>(x, M, L, d, modb, bs, so, co, hm, eps, out);
  }
#undef WAN_LN_CASE
  return hipGetLastError();
}

hipError_t launch_ln_mod(const float *x, int M, int L, int d, const float *modb, long modb_bstride,
                         int shift_off, int scale_off, int has_mod, float eps, void *out,
                         int out_f32, hipStream_t s) {
  if (out_f32)
    return ln_dispatch<float>(x, M, L, d, modb, modb_bstride, shift_off, scale_off, has_mod, eps,
                              (float *)out, s);
  return ln_dispatch<bf16>(x, M, L, d, modb, modb_bstride, shift_off, scale_off, has_mod, eps,
                           (bf16 *)out, s);
}

hipError_t launch_ln_mod_fp8(const float *x, int M, int L, int d, const float *modb,
                             long modb_bstride, int shift_off, int scale_off, int has_mod, float eps,
                             void *q, float *scale, hipStream_t s) {
  if (d % 256 || d / 256 > 24) return hipErrorInvalidValue;
  dim3 grid((M + 3) / 4), blk(256);
  uint8_t *qb = (uint8_t *)q;
#define WAN_LNQ_CASE(n)                                                                             \
  case n:                                                                                           \
    k_ln_mod_fp8<n><<<grid, blk, 0, s>>>(x, M, L, modb, modb_bstride, shift_off, scale_off, has_mod, \
                                         eps, qb, scale);                                           \
    break;
  switch (d / 256) {
    WAN_LNQ_CASE(1) WAN_LNQ_CASE(2) WAN_LNQ_CASE(3) WAN_LNQ_CASE(4) WAN_LNQ_CASE(5) WAN_LNQ_CASE(6)
    WAN_LNQ_CASE(8) WAN_LNQ_CASE(10) WAN_LNQ_CASE(12) WAN_LNQ_CASE(16) WAN_LNQ_CASE(20) WAN_LNQ_CASE(24)
    default: return hipErrorInvalidValue;
  }
#undef WAN_LNQ_CASE
  return hipGetLastError();
}

// widths the fused LayerNorm -> E4M3 kernel covers
bool ln_mod_fp8_supported(int d) {
  const int n = d / 256;
  return d % 256 == 0 && (n <= 6 || n == 8 || n == 10 || n == 12 || n == 16 || n == 20 || n == 24);
}

}  // namespace wan
