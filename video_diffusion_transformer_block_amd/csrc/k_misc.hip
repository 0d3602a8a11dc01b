// The small kernels around the blocks: the shared timestep MLP (sinusoid ->
// Linear -> SiLU -> Linear to six modulation vectors), the (1,2,2) patch
// gather that turns patchify into a GEMM, and the head Linear fused with the
// unpatchify scatter.
//   Timestep MLP: "Wan: Open and Advanced Large-Scale Video Generative Models
//   (Wan 2.1)", section Diffusion Transformer (one Linear+SiLU MLP shared by
//   all blocks predicts six modulation parameters) and table 配置表
//   (frequency dimension 256).
//   Patchify / unpatchify: same page, section Diffusion Transformer (3D
//   convolution with a (1,2,2) kernel; sequence length (1+T/4)*H/16*W/16).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace wan {

// e[b, k] = cos(t_b w_k) for k < half, sin(t_b w_{k-half}) after; w_k = 10000^(-k/half).
// Evaluated in double so the argument t*w (t up to 1000) keeps full precision.
__global__ void k_tsin(const float *__restrict__ t, int B, int fd, float *__restrict__ e) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * fd) return;
  int b = i / fd, k = i % fd, half = fd / 2;
  int kk = k < half ? k : k - half;
  double w = exp(-log(10000.0) * (double)kk / (double)half);
  double arg = (double)t[b] * w;
  e[i] = (float)(k < half ? cos(arg) : sin(arg));
}

// y[b, j] = act(sum_k W[j, k] x[b, k] + bias[j]) for every b < B (B <= 8):
// one wavefront per output row j, 16-byte weight loads, the x rows from cache.
template <typename T, int ACT>
__global__ __launch_bounds__(256) void k_gemv(const T *__restrict__ W, const T *__restrict__ bias,
                                              const float *__restrict__ x, int B, int N, int K,
                                              float *__restrict__ y) {
  constexpr int VW = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= N) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const T *wr = W + (long)j * K;
  for (int k0 = lane * VW; k0 < K; k0 += 64 * VW) {
    T wv[VW];
    if (k0 + VW <= K) {
      *reinterpret_cast<uint4 *>(wv) = ld16(wr + k0);
    } else {
#pragma unroll
      for (int u = 0; u < VW; ++u) wv[u] = k0 + u < K ? wr[k0 + u] : from_f<T>(0.f);
    }
    const bool full = k0 + VW <= K && (K & 3) == 0;
    for (int b = 0; b < B; ++b) {
      const float *xb = x + (long)b * K + k0;
      float xv[VW];
      if (full) {   // x rows are 16-byte aligned (K % 4 == 0): vector loads
#pragma unroll
        for (int u = 0; u < VW; u += 4) *reinterpret_cast<float4 *>(xv + u) = *reinterpret_cast<const float4 *>(xb + u);
      } else {
#pragma unroll
        for (int u = 0; u < VW; ++u) xv[u] = k0 + u < K ? xb[u] : 0.f;
      }
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < VW; ++u) s = fmaf(to_f<T>(wv[u]), xv[u], s);
      acc[b] += s;
    }
  }
  for (int b = 0; b < B; ++b) {
    float v = wave_sum(acc[b]) + (bias ? to_f<T>(bias[j]) : 0.f);
    if (ACT == 1) v = silu(v);
    if (lane == 0) y[(long)b * N + j] = v;
  }
}

template <typename T>
static void tmlp_go(const float *t, int B, int fd, int d, const void *w1, const void *b1,
                    const void *w2, const void *b2, float *hid, float *mod, hipStream_t s) {
  float *e = hid + (long)B * d;   // [B, fd] after the hidden vector
  k_tsin<<<(B * fd + 255) / 256, 256, 0, s>>>(t, B, fd, e);
  k_gemv<T, 1><<<(d + 3) / 4, 256, 0, s>>>((const T *)w1, (const T *)b1, e, B, d, fd, hid);
  k_gemv<T, 0><<<(6 * d + 3) / 4, 256, 0, s>>>((const T *)w2, (const T *)b2, hid, B, 6 * d, d, mod);
}

hipError_t launch_tmlp(const float *t, int B, int freq_dim, int d, const void *w1, const void *b1,
                       const void *w2, const void *b2, float *hidden, float *mod, int f32,
                       hipStream_t s) {
  if (B > 8) return hipErrorInvalidValue;
  if (f32) tmlp_go<float>(t, B, freq_dim, d, w1, b1, w2, b2, hidden, mod, s);
  else tmlp_go<bf16>(t, B, freq_dim, d, w1, b1, w2, b2, hidden, mod, s);
  return hipGetLastError();
}

// P[m, k] = latent[b, c, f, 2i+a, 2j+bb] with m = b*L + (f*Hp + i)*Wp + j and
// k = c*4 + a*2 + bb (the Conv3d weight order); columns 4C..Kp-1 are zero.
template <typename T>
__global__ void k_patch_gather(const float *__restrict__ lat, int B, int C, int F, int H8, int W8,
                               int Kp, T *__restrict__ P) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int Hp = H8 / 2, Wp = W8 / 2;
  const long L = (long)F * Hp * Wp;
  if (i >= B * L * Kp) return;
  const int k = i % Kp;
  const long m = i / Kp;
  float v = 0.f;
  if (k < 4 * C) {
    const int b = m / L;
    const long n = m % L;
    const int f = n / (Hp * Wp), rem = n % (Hp * Wp), ii = rem / Wp, jj = rem % Wp;
    const int c = k >> 2, aa = (k >> 1) & 1, bb = k & 1;
    v = lat[(((long)b * C + c) * F + f) * H8 * W8 + (long)(2 * ii + aa) * W8 + 2 * jj + bb];
  }
  P[i] = from_f<T>(v);
}

hipError_t launch_patch_gather(const float *latent, int B, int C, int F, int H8, int W8, int Kp,
                               void *P, int f32, hipStream_t s) {
  const long n = (long)B * F * (H8 / 2) * (W8 / 2) * Kp;
  const int blocks = (int)((n + 255) / 256);
  if (f32) k_patch_gather<float><<<blocks, 256, 0, s>>>(latent, B, C, F, H8, W8, Kp, (float *)P);
  else k_patch_gather<bf16><<<blocks, 256, 0, s>>>(latent, B, C, F, H8, W8, Kp, (bf16 *)P);
  return hipGetLastError();
}

// dst[r, 0..Kp) = src[r, 0..K) followed by zeros (weight rows padded to the GEMM K tile)
template <typename T>
__global__ void k_pad_rows(const T *__restrict__ src, int R, int K, int Kp, T *__restrict__ dst) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * Kp) return;
  const int k = i % Kp;
  const long r = i / Kp;
  dst[i] = k < K ? src[r * K + k] : from_f<T>(0.f);
}

hipError_t launch_pad_rows(const void *src, int R, int K, int Kp, void *dst, int f32, hipStream_t s) {
  const long n = (long)R * Kp;
  const int blocks = (int)((n + 255) / 256);
  if (f32) k_pad_rows<float><<<blocks, 256, 0, s>>>((const float *)src, R, K, Kp, (float *)dst);
  else k_pad_rows<bf16><<<blocks, 256, 0, s>>>((const bf16 *)src, R, K, Kp, (bf16 *)dst);
  return hipGetLastError();
}

// out[b, c, f, 2i+a, 2j+bb] = sum_k x[m, k] W[c*4+a*2+bb, k] + bias   (float32 math;
// x is the float32 residual stream).  64 tokens x 64 outputs per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void k_head_unpatch(const float *__restrict__ x, int M, int L,
                                                      int F, int Hp, int Wp, int d,
                                                      const T *__restrict__ W,
                                                      const T *__restrict__ bias, int NO,
                                                      float *__restrict__ out) {
  __shared__ float sx[16][68], sw[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_m = (M + 63) / 64;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * 64, n0 = tn * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, r = idx >> 4, kk = idx & 15;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      sx[kk][r] = (gm < M && gk < d) ? x[(long)gm * d + gk] : 0.f;
      sw[kk][r] = (gn < NO && gk < d) ? to_f<T>(W[(long)gn * d + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = sx[kk][ty * 4 + i]; bv[i] = sw[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(av[i], bv[jj], acc[i][jj]);
    }
    __syncthreads();
  }
  const int H8 = 2 * Hp, W8 = 2 * Wp, C = NO / 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    const int b = m / L, n = m % L;
    const int f = n / (Hp * Wp), rem = n % (Hp * Wp), ii = rem / Wp, jj2 = rem % Wp;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int o = n0 + tx * 4 + jj;
      if (o >= NO) continue;
      const int c = o >> 2, aa = (o >> 1) & 1, bb = o & 1;
      const float v = acc[i][jj] + (bias ? to_f<T>(bias[o]) : 0.f);
      out[(((long)b * C + c) * F + f) * H8 * W8 + (long)(2 * ii + aa) * W8 + 2 * jj2 + bb] = v;
    }
  }
}

// bf16 weights: the head is a skinny GEMM (N = 4*out_ch outputs, K = d), bound
// by reading the float32 stream once.  A workgroup owns 32 tokens; its four
// wavefronts split K, each lane rounds its x values to bf16 in registers
// (the operand rounding of every GEMM here) and feeds
// v_mfma_f32_32x32x16_bf16 with weight rows straight from L2; the four
// partial 32 x N tiles are added through LDS and scattered by the unpatchify
// rule, bias added.
template <int NB>   // N = 32 * NB outputs
__global__ __launch_bounds__(256) void k_head_mfma(const float *__restrict__ x, int M, int L, int F,
                                                   int Hp, int Wp, int d, const bf16 *__restrict__ W,
                                                   const bf16 *__restrict__ bias,
                                                   float *__restrict__ out) {
  __shared__ float part[4][NB * 16][64];   // [wave][register][lane]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const long m0 = (long)blockIdx.x * 32;
  const long row = m0 + l32 < M ? m0 + l32 : M - 1;   // tail rows read a valid row, never stored
  const int kw = d / 4, kbeg = w * kw;                 // this wavefront's K range
  const float *xp = x + row * d + kbeg + g * 8;
  const bf16 *wp = W + (long)l32 * d + kbeg + g * 8;
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
#pragma unroll 4
  for (int k = 0; k < kw; k += 16) {
    const float4 u0 = *reinterpret_cast<const float4 *>(xp + k);
    const float4 u1 = *reinterpret_cast<const float4 *>(xp + k + 4);
    bf16x8 a;
    a[0] = f2bf(u0.x); a[1] = f2bf(u0.y); a[2] = f2bf(u0.z); a[3] = f2bf(u0.w);
    a[4] = f2bf(u1.x); a[5] = f2bf(u1.y); a[6] = f2bf(u1.z); a[7] = f2bf(u1.w);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8 *>(wp + (long)nb * 32 * d + k);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[w][nb * 16 + r][lane] = acc[nb][r];
  __syncthreads();
  // lane (g, l32), register r of block nb holds token row (r/4)*8 + g*4 + r%4, output nb*32 + l32
  const int H8 = 2 * Hp, W8 = 2 * Wp, C = NB * 8;
  for (int i = threadIdx.x; i < NB * 16 * 64; i += 256) {
    const int reg = i >> 6, ln = i & 63, nb = reg >> 4, r = reg & 15;
    const long m = m0 + (r >> 2) * 8 + (ln >> 5) * 4 + (r & 3);
    if (m >= M) continue;
    const int o = nb * 32 + (ln & 31);
    float v = part[0][reg][ln] + part[1][reg][ln] + part[2][reg][ln] + part[3][reg][ln];
    if (bias) v += (float)bias[o];
    const long bq = m / L, n = m % L;
    const int f = (int)(n / (Hp * Wp)), rem = (int)(n % (Hp * Wp)), ii = rem / Wp, jj = rem % Wp;
    const int c = o >> 2, aa = (o >> 1) & 1, bb = o & 1;
    out[((bq * C + c) * F + f) * (long)H8 * W8 + (long)(2 * ii + aa) * W8 + 2 * jj + bb] = v;
  }
}

hipError_t launch_head_unpatchify(const float *x, int B, int F, int Hp, int Wp, int d,
                                  const void *w, const void *b, int out_ch, float *out, int f32,
                                  hipStream_t s) {
  const int L = F * Hp * Wp, M = B * L, NO = out_ch * 4;
  const int blocks = ((M + 63) / 64) * ((NO + 63) / 64);
  if (!f32 && d % 64 == 0 && (NO == 32 || NO == 64)) {
    const int wgs = (M + 31) / 32;
    if (NO == 64)
      k_head_mfma<2><<<wgs, 256, 0, s>>>(x, M, L, F, Hp, Wp, d, (const bf16 *)w, (const bf16 *)b, out);
    else
      k_head_mfma<1><<<wgs, 256, 0, s>>>(x, M, L, F, Hp, Wp, d, (const bf16 *)w, (const bf16 *)b, out);
    return hipGetLastError();
  }
  if (f32)
    k_head_unpatch<float><<<blocks, 256, 0, s>>>(x, M, L, F, Hp, Wp, d, (const float *)w,
                                                  (const float *)b, NO, out);
  else
    k_head_unpatch<bf16><<<blocks, 256, 0, s>>>(x, M, L, F, Hp, Wp, d, (const bf16 *)w,
                                                 (const bf16 *)b, NO, out);
  return hipGetLastError();
}

// ---- sampler ("Wan: Open and Advanced Large-Scale Video Generative Models
// (Wan 2.1)", section 训练方法: the flow x_tau = tau x1 + (1 - tau) x0 with
// velocity x1 - x0, integrated here by explicit Euler steps; "Wan 2.1 AI：下一代
// 开源视频生成技术的突破性实践", section 工作原理: the guidance scale)

__global__ void k_fill(float *__restrict__ p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill(float *p, int n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// x += dt * v on channels 0..out_ch-1 of every sample (latent [B, in_ch,
// plane], velocity [B, out_ch, plane]).  guided: B == 2, sample 0 is the
// conditional and sample 1 the unconditional prediction for the same latent;
// both samples receive x0 + dt * (v1 + s (v0 - v1)).
__global__ __launch_bounds__(256) void k_euler(float *__restrict__ lat, const float *__restrict__ vel,
                                               int B, int in_ch, int out_ch, long plane, float dt,
                                               int guided, float scale) {
  const long n = (long)out_ch * plane;   // moving elements per sample
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const long ls = (long)in_ch * plane;   // latent sample stride
  if (guided) {
    const float vc = vel[e], vu = vel[n + e];
    const float v = vu + scale * (vc - vu);
    const float x = lat[e] + dt * v;
    lat[e] = x;
    lat[ls + e] = x;
  } else {
    for (int b = 0; b < B; ++b) lat[b * ls + e] += dt * vel[b * n + e];
  }
}

hipError_t launch_euler(float *lat, const float *vel, int B, int in_ch, int out_ch, long plane,
                        float dt, int guided, float scale, hipStream_t s) {
  const long n = (long)out_ch * plane;
  if (n <= 0) return hipSuccess;
  k_euler<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(lat, vel, B, in_ch, out_ch, plane, dt, guided,
                                                      scale);
  return hipGetLastError();
}

}  // namespace wan
