// GEMMs of the DiT block: C[M,N] = A[M,K] . B[N,K]^T (+ bias) with fused
// epilogues (bf16 store, float32 store, tanh-GELU, gated residual add into
// the float32 stream).  These are the block's Linear layers: QKV, the
// attention out-projections, the cross-attention Q/K/V projections, the FFN
// ("Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)",
// table 配置表 for the widths), patchify as a GEMM over gathered patches.
//
// bf16 path: 256x256x64 block tile, 4 wavefronts in a 2x2 grid, each owning a
// 128x128 tile of 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per
// lane).  A and B tiles are staged through LDS with a 16-byte-chunk XOR
// swizzle so that the 32 rows an MFMA operand read touches land in distinct
// banks; global loads for the next K tile are in flight while the current
// one is multiplied (two LDS stages, one barrier per K tile).
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

constexpr int GBM = 256, GBN = 256, GBK = 64;

WAN_DEV int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int KIND, bool BROWS, typename T>
WAN_DEV void epi_one(const GemmDesc &g, int m, int n, float v) {
  if (g.bias) v += to_f<T>(reinterpret_cast<const T *>(g.bias)[BROWS ? m : n]);
  if (KIND == OUT_BF16) {
    reinterpret_cast<T *>(g.C)[(long)m * g.ldc + n] = from_f<T>(v);
  } else if (KIND == OUT_F32) {
    reinterpret_cast<float *>(g.C)[(long)m * g.ldc + n] = v;
  } else if (KIND == OUT_GELU) {
    reinterpret_cast<T *>(g.C)[(long)m * g.ldc + n] = from_f<T>(gelu_tanh(v));
  } else {  // OUT_RESID
    float gt = 1.0f;
    if (g.gate) gt = g.gate[(long)(m / g.rows_per_batch) * g.gate_bstride + n];
    float *xp = g.X + (long)m * g.ldx + n;
    *xp = *xp + gt * v;
  }
}

template <int KIND, bool BROWS>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(GemmDesc g) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][GBM * GBK];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][GBN * GBK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int tiles_m = (g.M + GBM - 1) / GBM;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  // consecutive logical tiles walk down M inside one N column strip, so the
  // tiles resident on one XCD share their B (weight) strip in L2
  const int tn = bid / tiles_m, tm = bid % tiles_m;
  (void)tiles_n;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const bf16 *A = reinterpret_cast<const bf16 *>(g.A);
  const bf16 *Bm = reinterpret_cast<const bf16 *>(g.B);

  // global -> register staging: 8 chunks of A and 8 of B per thread
  const int lrow = tid >> 3, lc = tid & 7;
  uint4 ra[8], rb[8];
  auto gload = [&](int kt) {
    const int k0 = kt * GBK + lc * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = lrow + 32 * i;
      int gm = m0 + r, gn = n0 + r;
      ra[i] = gm < g.M ? ld16(A + (long)gm * g.lda + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = gn < g.N ? ld16(Bm + (long)gn * g.ldb + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = lrow + 32 * i;
      int off = r * GBK + ((lc ^ swz8(r)) * 8);
      st16(&sA[st][off], ra[i]);
      st16(&sB[st][off], rb[i]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.K / GBK;
  gload(0);
  sstore(0);
  __syncthreads();

  const int arow0 = wm * 128 + (lane & 31);
  const int brow0 = wn * 128 + (lane & 31);
  const int half = lane >> 5;

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks * 2 + half;
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = arow0 + i * 32;
        a[i] = *reinterpret_cast<const bf16x8 *>(&sA[st][r * GBK + ((c ^ swz8(r)) * 8)]);
        int q = brow0 + i * 32;
        b[i] = *reinterpret_cast<const bf16x8 *>(&sB[st][q * GBK + ((c ^ swz8(q)) * 8)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[row = (r/4)*8 + half*4 + r%4][col = lane%32] of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 128 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        if (m < g.M) epi_one<KIND, BROWS, bf16>(g, m, n, acc[i][j][r]);
      }
    }
}

// float32 path (small fp32 workloads): 64x64 tile, 4x4 outputs per thread.
template <int KIND, bool BROWS>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmDesc g) {
  __shared__ float sA[16][68], sB[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_m = (g.M + 63) / 64;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * 64, n0 = tn * 64;
  const float *A = reinterpret_cast<const float *>(g.A);
  const float *Bm = reinterpret_cast<const float *>(g.B);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + 256 * i;       // 0..1023: row = idx/16, k = idx%16
      int r = idx >> 4, kk = idx & 15;
      int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      sA[kk][r] = (gm < g.M && gk < g.K) ? A[(long)gm * g.lda + gk] : 0.f;
      sB[kk][r] = (gn < g.N && gk < g.K) ? Bm[(long)gn * g.ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[kk][ty * 4 + i]; b[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < g.M && n < g.N) epi_one<KIND, BROWS, float>(g, m, n, acc[i][j]);
    }
}

template <int KIND, bool BROWS>
static void gemm_go(const GemmDesc &g, hipStream_t s) {
  if (g.f32) {
    int blocks = ((g.M + 63) / 64) * ((g.N + 63) / 64);
    k_gemm_f32<KIND, BROWS><<<blocks, 256, 0, s>>>(g);
  } else {
    int blocks = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
    k_gemm_bf16<KIND, BROWS><<<blocks, 256, 0, s>>>(g);
  }
}

hipError_t launch_gemm(const GemmDesc &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (!g.f32 && (g.K % GBK)) return hipErrorInvalidValue;
  const bool br = g.bias_rows != 0;
  switch (g.kind) {
    case OUT_BF16: br ? gemm_go<OUT_BF16, true>(g, s) : gemm_go<OUT_BF16, false>(g, s); break;
    case OUT_F32: gemm_go<OUT_F32, false>(g, s); break;
    case OUT_GELU: gemm_go<OUT_GELU, false>(g, s); break;
    case OUT_RESID: gemm_go<OUT_RESID, false>(g, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace wan
