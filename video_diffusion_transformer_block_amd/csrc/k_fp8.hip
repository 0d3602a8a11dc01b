// FP8 quantisation for the FP8 GEMM ("Wan: Open and Advanced Large-Scale Video
// Generative Models (Wan 2.1)", section Infra / 推理优化: FP8 GEMM with
// per-tensor weight scales and per-token activation scales).
//
// Format: OCP E4M3 (v_cvt_pk_fp8_f32 on gfx950: round to nearest even, no
// saturation -- inputs are clamped to +-448 first).  A scale maps the largest
// magnitude to 448: inv = 448 / amax (correctly rounded float32 division),
// code = E4M3(clamp(x * inv)), stored scale = amax / 448 (x ~= code * scale);
// an all-zero row or tensor gets scale 1.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

WAN_DEV float inv_scale(float amax) { return amax > 0.f ? 448.0f / amax : 1.0f; }
WAN_DEV float deq_scale(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

// two floats -> two E4M3 bytes (low byte first)
WAN_DEV unsigned short pack2(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (unsigned short)(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFF);
}

// 8 bf16 -> 8 E4M3 bytes scaled by inv
WAN_DEV uint2 quant8(const uint4 &u, float inv) {
  const bf16 *e = reinterpret_cast<const bf16 *>(&u);
  uint2 r;
  r.x = pack2((float)e[0] * inv, (float)e[1] * inv) | ((unsigned)pack2((float)e[2] * inv, (float)e[3] * inv) << 16);
  r.y = pack2((float)e[4] * inv, (float)e[5] * inv) | ((unsigned)pack2((float)e[6] * inv, (float)e[7] * inv) << 16);
  return r;
}

WAN_DEV float amax8(const uint4 &u, float m) {
  const bf16 *e = reinterpret_cast<const bf16 *>(&u);
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)e[i]));
  return m;
}

// one wavefront per row; K % 8 == 0, rows 16-byte aligned (ldx % 8 == 0, ldq % 8 == 0)
__global__ __launch_bounds__(256) void k_quant_rows(const bf16 *__restrict__ x, int M, int K, long ldx,
                                                    uint8_t *__restrict__ q, long ldq,
                                                    float *__restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const bf16 *xr = x + row * ldx;
  float m = 0.f;
  for (int c = lane * 8; c < K; c += 512) m = amax8(ld16(xr + c), m);
  m = wave_max(m);
  const float inv = inv_scale(m);
  uint8_t *qr = q + row * ldq;
  for (int c = lane * 8; c < K; c += 512)
    *reinterpret_cast<uint2 *>(qr + c) = quant8(ld16(xr + c), inv);
  if (lane == 0) scale[row] = deq_scale(m);
}

hipError_t launch_quant_rows_fp8(const void *x, int M, int K, long ldx, void *q, long ldq,
                                 float *scale, hipStream_t s) {
  if (M <= 0 || K <= 0) return hipSuccess;
  k_quant_rows<<<(M + 3) / 4, 256, 0, s>>>((const bf16 *)x, M, K, ldx, (uint8_t *)q, ldq, scale);
  return hipGetLastError();
}

// per-tensor: amax over n elements (n % 8 == 0) by an atomic max on the float
// bits (non-negative floats order as unsigned integers), then the cast
__global__ void k_zero_u32(unsigned *p) { *p = 0u; }

__global__ __launch_bounds__(256) void k_amax(const bf16 *__restrict__ w, long n8,
                                              unsigned *__restrict__ amax_bits) {
  float m = 0.f;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256)
    m = amax8(ld16(w + i * 8), m);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __float_as_uint(m));
}

__global__ __launch_bounds__(256) void k_quant_tensor(const bf16 *__restrict__ w, long n8,
                                                      const unsigned *__restrict__ amax_bits,
                                                      uint8_t *__restrict__ q, float *__restrict__ scale) {
  const float m = __uint_as_float(*amax_bits);
  const float inv = inv_scale(m);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256)
    *reinterpret_cast<uint2 *>(q + i * 8) = quant8(ld16(w + i * 8), inv);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = deq_scale(m);
}

hipError_t launch_quant_tensor_fp8(const void *w, long n, void *q, float *scale, unsigned *amax_bits,
                                   hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long n8 = n / 8;
  const int blocks = (int)(n8 / 256 + 1 < 2048 ? n8 / 256 + 1 : 2048);
  k_zero_u32<<<1, 1, 0, s>>>(amax_bits);
  k_amax<<<blocks, 256, 0, s>>>((const bf16 *)w, n8, amax_bits);
  k_quant_tensor<<<blocks, 256, 0, s>>>((const bf16 *)w, n8, amax_bits, (uint8_t *)q, scale);
  return hipGetLastError();
}

}  // namespace wan
