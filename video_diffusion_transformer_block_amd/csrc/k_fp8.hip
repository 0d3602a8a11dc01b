// Per-token and per-tensor FP8 (OCP E4M3) quantisation for the FP8 GEMM
// ("Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)",
// section Infra / 推理优化: FP8 GEMM with per-tensor weight scales and
// per-token activation scales); format and scale rule in fp8.hpp.
#include "fp8.hpp"
#include "kernels.hpp"

namespace wan {

// one wavefront per row with the row held in registers (at most NC 16-byte
// chunks per lane: K <= NC * 512): one read of the row, then the codes
template <int NC>
__global__ __launch_bounds__(256) void k_quant_rows_reg(const bf16 *__restrict__ x, int M, int K,
                                                        long ldx, uint8_t *__restrict__ q, long ldq,
                                                        float *__restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const bf16 *xr = x + row * ldx;
  uint4 v[NC];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (i * 64 + lane) * 8;
    v[i] = c < K ? ld16(xr + c) : make_uint4(0, 0, 0, 0);
    m = amax8(v[i], m);
  }
  m = wave_max(m);
  const float inv = inv_scale(m);
  uint8_t *qr = q + row * ldq;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (i * 64 + lane) * 8;
    if (c < K) *reinterpret_cast<uint2 *>(qr + c) = quant8(v[i], inv);
  }
  if (lane == 0) scale[row] = deq_scale(m);
}

// wider rows: two passes over the row (maximum, then codes)
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
  const int grid = (M + 3) / 4;
  const bf16 *xb = (const bf16 *)x;
  uint8_t *qb = (uint8_t *)q;
  if (K <= 4 * 512) k_quant_rows_reg<4><<<grid, 256, 0, s>>>(xb, M, K, ldx, qb, ldq, scale);
  else if (K <= 8 * 512) k_quant_rows_reg<8><<<grid, 256, 0, s>>>(xb, M, K, ldx, qb, ldq, scale);
  else if (K <= 18 * 512) k_quant_rows_reg<18><<<grid, 256, 0, s>>>(xb, M, K, ldx, qb, ldq, scale);
  else k_quant_rows<<<grid, 256, 0, s>>>(xb, M, K, ldx, qb, ldq, scale);
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
