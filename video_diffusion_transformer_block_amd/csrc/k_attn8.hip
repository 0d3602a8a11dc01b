// 8-bit attention ("Wan: Open and Advanced Large-Scale Video Generative Models
// (Wan 2.1)", section Infra / 推理优化: 8-bit FlashAttention with Int8 for
// S = QK^T, FP8 for O = PV and FP32 accumulation across key blocks).
//
// Quantisers (HBM-bound, every group read once, codes decided in float32):
//  * q per token and head (128 features) to Int8: inv = 127 / amax (correctly
//    rounded), code = round-half-even(clamp(x * inv, +-127)), scale = amax / 127;
//  * k per block of 64 keys and head (64 x 128 values), the same rule;
//  * V^T per channel (one row of V^T: one head feature over the keys) to OCP
//    E4M3 with scale amax / 448 (the FP8 GEMM's rule); columns Lk ..
//    round_up(Lk, 64)-1 of each batch segment are written as zeros.
// An all-zero group gets scale 1.
//
// Attention, hd = 128, the bf16 kernel's workgroup shape (256 queries of one
// (batch, head), eight wavefronts of 32 queries, two per SIMD, transposed
// scores S^T = K Q^T so that a lane holds keys of ONE query):
//  * scores with v_mfma_i32_32x32x32_i8, four per 32-key block.  The int32
//    accumulator starts at the bit pattern of 1.5 * 2^23, so the result read
//    as a float is exactly 1.5 * 2^23 + S (|S| <= 128 * 127^2 < 2^22); one
//    FMA, f * c + bb with c = sq sk log2(e)/sqrt(hd) and bb = -(1.5 * 2^23 c
//    + m), gives the score in log2 units minus the running max m;
//  * probabilities p = exp2 of that: 2^7 at a freshly set max.  The max is
//    taken from the first tile and raised, by a whole number of log2 units,
//    only when a probability of a tile would pass 448, E4M3's largest value
//    (a lane max of the tile's scores, checked before the exponentials).
//    The accumulators are not rescaled: O and the row sums stay referred to
//    the first max, 2^64 below it, and each tile's probabilities enter them
//    times 2^E, E the total rise so far, through the E8M0 scale of the B
//    operand of the MFMAs.  Should E pass 150 the accumulated terms weigh
//    less than 2^-130 against the new ones and are cleared;
//  * P^T in E4M3 is the B operand of O^T += V^T P^T
//    (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales).  The rows of a K
//    tile sit in LDS in a permuted order (ksig8) that makes a lane's 32 score
//    registers the probabilities of 32 consecutive keys, so a V^T fragment is
//    32 consecutive bytes of a V^T row;
//  * the row sums come from one more MFMA of the same P^T registers, a
//    16x16x128 one whose A operand holds ones and zeros per lane: it adds a
//    query's 64 probabilities (with unit scales -- a K block of that MFMA
//    mixes two queries, whose E may differ), and the lane adds it times 2^E
//    to its float32 sum: the normaliser is exactly the sum of the rounded
//    weights the PV MFMAs use;
//  * software pipeline: iteration j runs the score MFMAs of tile j+1 and the
//    PV MFMAs of tile j-1 while the vector unit turns the scores of tile j
//    into probabilities; K and V^T tiles of 64 keys go global -> LDS directly
//    (double-buffered, XOR-swizzled 16-byte chunks); one barrier per tile.
#include <type_traits>

#include "attn8.hpp"
#include "common.hpp"
#include "fp8.hpp"

namespace wan {

namespace {

constexpr int QW8 = 256;      // queries per workgroup
constexpr int KT8 = 64;       // keys per tile = keys per K quantisation block
constexpr int HD8 = 128;      // head dim
constexpr float XMAX8 = 8.8f;       // exp2(8.8) = 445.7 <= 448: the largest exponent E4M3 holds
constexpr float XTOP8 = 7.0f;       // a (re)set max puts the largest probability at 2^7
constexpr float K0F = 12582912.0f;  // 1.5 * 2^23
constexpr int K0I = 0x4B400000;     // its bit pattern

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void *lds_ptr8;

// LDS row R of a K tile holds key ksig8(R) of the tile.  Score register r of
// 32-key block kb in a lane of half g belongs to LDS row kb*32 + 8(r/4) +
// 4g + r%4 (the MFMA's accumulator layout); with this permutation that is key
// 32g + 16kb + r.
WAN_DEV int ksig8(int R) {
  return (((R >> 2) & 1) << 5) | (((R >> 5) & 1) << 4) | (((R >> 3) & 3) << 2) | (R & 3);
}
WAN_DEV int kswz8(int row) { return (row >> 1) & 7; }   // 128-byte rows: 8 chunks
WAN_DEV int vswz8(int row) { return (row >> 2) & 3; }   // 64-byte rows: 4 chunks

WAN_DEV float half_swap(float v) { return __shfl_xor(v, 32); }

// eight bf16 -> eight Int8 codes (x * inv, clamp, round half to even)
WAN_DEV uint2 quant8_i8(const uint4 &u, float inv) {
  const bf16 *e = reinterpret_cast<const bf16 *>(&u);
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = __builtin_rintf(fminf(fmaxf((float)e[i] * inv, -127.0f), 127.0f));
    w[i >> 2] |= ((unsigned)(int)v & 0xFFu) << (8 * (i & 3));
  }
  return make_uint2(w[0], w[1]);
}

WAN_DEV float i8_inv(float amax) { return amax > 0.f ? 127.0f / amax : 1.0f; }
WAN_DEV float i8_scale(float amax) { return amax > 0.f ? amax / 127.0f : 1.0f; }

// ---- quantisers ----------------------------------------------------------

// q: one (token, head) group per 16 lanes, 8 features per lane
__global__ __launch_bounds__(256) void k_quant_q8(const bf16 *q, long ldq, int rows, int H,
                                                  int8_t *q8, long ldq8, float *qs) {
  const long gidx = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const bool ok = gidx < (long)rows * H;
  const long row = ok ? gidx / H : 0;
  const int h = ok ? (int)(gidx % H) : 0;
  const uint4 u = ok ? ld16(q + row * ldq + h * HD8 + c * 8) : make_uint4(0, 0, 0, 0);
  float m = amax8(u, 0.f);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (!ok) return;
  *reinterpret_cast<uint2 *>(q8 + row * ldq8 + h * HD8 + c * 8) = quant8_i8(u, i8_inv(m));
  if (c == 0) qs[row * H + h] = i8_scale(m);
}

// k: one (batch, head, 64-key block) per workgroup; thread t holds chunk t%16
// of key rows t/16 + 16 i, i = 0..3
__global__ __launch_bounds__(256) void k_quant_k8(const bf16 *k, long ldk, int B, int H, int Lk,
                                                  int8_t *k8, long ldk8, float *ks) {
  __shared__ float red[4];
  const int nkb = (Lk + KT8 - 1) / KT8;
  const int kb = blockIdx.x % nkb, bh = blockIdx.x / nkb;
  const int h = bh % H, b = bh / H;
  const int c = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  uint4 u[4];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kb * KT8 + r0 + 16 * i;
    u[i] = key < Lk ? ld16(k + ((long)b * Lk + key) * ldk + h * HD8 + c * 8) : make_uint4(0, 0, 0, 0);
    m = amax8(u[i], m);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = i8_inv(m);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kb * KT8 + r0 + 16 * i;
    if (key < Lk)
      *reinterpret_cast<uint2 *>(k8 + ((long)b * Lk + key) * ldk8 + h * HD8 + c * 8) = quant8_i8(u[i], inv);
  }
  if (threadIdx.x == 0) ks[(long)bh * nkb + kb] = i8_scale(m);
}

// V^T: one (batch, row) per workgroup; two passes over the row (the second
// from L2).  The caller's padding columns Lk .. round_up(Lk, 64)-1 exist and
// are read, their values masked.
__global__ __launch_bounds__(256) void k_quant_vt8(const bf16 *vt, long ldv, long vt_bstride, int H, int Lk,
                                                   uint8_t *v8t, long ldv8, long v8_bstride, float *vs) {
  __shared__ float red[4];
  const int nrow = H * HD8;
  const int row = blockIdx.x % nrow, b = blockIdx.x / nrow;
  const int Lkp = (Lk + KT8 - 1) / KT8 * KT8;
  const bf16 *src = vt + (long)row * ldv + (long)b * vt_bstride;
  uint8_t *dst = v8t + (long)row * ldv8 + (long)b * v8_bstride;
  auto masked = [&](int j0) {
    uint4 u = ld16(src + j0);
    if (j0 + 8 > Lk) {
      bf16 *e = reinterpret_cast<bf16 *>(&u);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i >= Lk) e[i] = (bf16)0.f;
    }
    return u;
  };
  float m = 0.f;
  for (int j0 = threadIdx.x * 8; j0 < Lkp; j0 += 256 * 8) m = amax8(masked(j0), m);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = inv_scale(m);
  for (int j0 = threadIdx.x * 8; j0 < Lkp; j0 += 256 * 8)
    *reinterpret_cast<uint2 *>(dst + j0) = quant8(masked(j0), inv);
  if (threadIdx.x == 0) vs[(long)b * nrow + row] = deq_scale(m);
}

// ---- attention -------------------------------------------------------------

__global__ __launch_bounds__(512, 1) void k_attn_i8f8(Attn8Desc a) {
  // one LDS variable per stage (separate alias scopes; see the bf16 kernel)
  __shared__ __attribute__((aligned(16))) uint8_t sK0[KT8 * HD8];   // [row][128 B], chunk ^ kswz8(row)
  __shared__ __attribute__((aligned(16))) uint8_t sK1[KT8 * HD8];
  __shared__ __attribute__((aligned(16))) uint8_t sV0[HD8 * KT8];   // [hd][64 B], chunk ^ vswz8(hd)
  __shared__ __attribute__((aligned(16))) uint8_t sV1[HD8 * KT8];
  auto kbuf = [&](auto P) -> const uint8_t * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sK1 : sK0;
    else if constexpr (decltype(P)::value == 0) return sK0;
    else return sK1;
  };
  auto vbuf = [&](auto P) -> const uint8_t * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sV1 : sV0;
    else if constexpr (decltype(P)::value == 0) return sV0;
    else return sV1;
  };
  auto kdst = [&](auto P) -> uint8_t * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sK1 : sK0;
    else if constexpr (decltype(P)::value == 0) return sK0;
    else return sK1;
  };
  auto vdst = [&](auto P) -> uint8_t * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sV1 : sV0;
    else if constexpr (decltype(P)::value == 0) return sV0;
    else return sV1;
  };
  auto other = [](auto P) {
    if constexpr (std::is_integral_v<decltype(P)>) return 1 - P;
    else return std::integral_constant<int, 1 - decltype(P)::value>{};
  };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int Lq = a.Lq, Lk = a.Lk, H = a.H;
  const int nqt = (Lq + QW8 - 1) / QW8;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = bid % nqt, bh = bid / nqt;
  const int h = bh % H, b = bh / H;
  const int ntiles = (Lk + KT8 - 1) / KT8;
  const float *ksp = a.ks + (long)bh * ntiles;

  // ---- Q fragments (B operand of S^T = K Q^T): MFMA st covers features
  // 32 st .. +32; lane half g holds bytes 32 st + 16 g .. +16 of its query
  const int qrow = qt * QW8 + w * 32 + l32;
  const bool qok = qrow < Lq;
  i32x4 qf[4];
  {
    const int8_t *qp = a.q8 + (long)(b * Lq + (qok ? qrow : 0)) * a.ldq8 + h * HD8 + g * 16;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint4 v = qok ? ld16(qp + st * 32) : make_uint4(0, 0, 0, 0);
      qf[st] = *reinterpret_cast<const i32x4 *>(&v);
    }
  }
  // log2 units per integer score unit, before the K block scale
  const float cq = (qok ? a.qs[(long)(b * Lq + qrow) * H + h] : 1.0f) * a.alpha;

  // ---- tile loaders.  K tile: 8 blocks of 1 KB (8 rows of 128 B); wavefront
  // w fills block w: lane i lands at row 8w + i/8, physical chunk i%8, and
  // fetches key ksig8(row), logical chunk (i%8) ^ kswz8(row).  Rows past Lk
  // read as zero (the descriptor spans this batch's keys).
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.k8 + (long)b * Lk * a.ldk8), 0, (int)((unsigned)Lk * (unsigned)a.ldk8), 0x00020000);
  int kgo;
  {
    const int row = w * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ kswz8(row);
    kgo = ksig8(row) * (int)a.ldk8 + h * HD8 + chunk * 16;
  }
  auto gloadK = [&](int j, auto P) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr8)(kdst(P) + w * 1024), 16,
                                             kgo + j * KT8 * (int)a.ldk8, 0, 0, 0);
  };
  // V^T tile: 8 blocks of 1 KB (16 rows of 64 B); wavefront w fills block w:
  // lane i lands at row 16w + i/4, physical chunk i%4, and fetches keys
  // 16 ((i%4) ^ vswz8(row)) .. +16 of the tile
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.v8t, 0, (int)((unsigned)(H * HD8) * (unsigned)a.ldv8), 0x00020000);
  int vgo;
  {
    const int row = w * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ vswz8(row);
    vgo = (h * HD8 + row) * (int)a.ldv8 + b * (int)a.v8_bstride + chunk * 16;
  }
  auto gloadV = [&](int j, auto P) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr8)(vdst(P) + w * 1024), 16, vgo + j * KT8, 0, 0, 0);
  };

  // LDS fragment offsets (bytes); the swizzles depend only on l32 (block
  // offsets are multiples of 32 rows)
  int koff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) koff[st] = l32 * HD8 + (((2 * st + g) ^ kswz8(l32)) * 16);
  int voff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) voff[e] = l32 * KT8 + (((2 * g + e) ^ vswz8(l32)) * 16);

  i32x16 kinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) kinit[r] = K0I;
  // A operand of the row-sum MFMA (16x16x128): lane l holds row l%16, key
  // group l/16 of the B operand -- the P^T registers read as 16 columns x 4
  // groups of 32 keys: group 0 = query c, keys 0-31; 1 = query c+16, keys
  // 0-31; 2 = query c, keys 32-63; 3 = query c+16, keys 32-63 (c = l%16).
  // Rows r with (r/4) even sum groups 0 and 2 (query c), the others groups 1
  // and 3 (query c+16); result row 4(l/16) + i then holds the row sum of
  // query l%32 in every lane.  E4M3 1.0 is 0x38.
  i32x8 ones;
  {
    const int sel = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838 : 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) ones[r] = sel;
  }

  f32x16 o[4];
  float lsum = 0.f;   // row sum of this lane's query, same reference as O
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t][r] = 0.f;
  }

  // biased integer scores of a tile (two 32-key blocks)
  auto qk = [&](const uint8_t *sk, i32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const i32x4 ka = *reinterpret_cast<const i32x4 *>(sk + kb * 32 * HD8 + koff[st]);
        s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qf[st], st ? s[kb] : kinit, 0, 0, 0);
      }
  };
  // exponents x = score (log2 units) - m of a tile; keys past Lk -> -inf
  auto expo = [&](const i32x16 (&s)[2], float c, float bb, bool ragged, int j, float (&x)[2][16]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kb][r] = fmaf(__int_as_float(s[kb][r]), c, bb);
    if (ragged) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j * KT8 + 32 * g + 16 * kb + r >= Lk) x[kb][r] = -INFINITY;
    }
  };
  // lane max of a tile's biased integer scores read as floats (positive,
  // ordered like the scores); keys past Lk count as the lowest score
  auto rawmax = [&](const i32x16 (&s)[2], bool ragged, int j) {
    float mx = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool dead = ragged && j * KT8 + 32 * g + 16 * kb + r >= Lk;
        mx = fmaxf(mx, dead ? 0.f : __int_as_float(s[kb][r]));
      }
    return mx;
  };
  auto lanemax = [&](const float (&x)[2][16]) {
    float m = x[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, x[kb][r]);
    return m;
  };
  // E4M3 probabilities in the B-operand layout: byte 16 kb + r = key 32 g + 16
  // kb + r.  The two packs of a dword write its low and its high half, so the
  // first starts from the register's old contents (no zeroing move).
  auto probs = [&](const float (&x)[2][16], i32x8 &p) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(x[kb][4 * q]),
                                                __builtin_amdgcn_exp2f(x[kb][4 * q + 1]), p[kb * 4 + q], false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(x[kb][4 * q + 2]),
                                            __builtin_amdgcn_exp2f(x[kb][4 * q + 3]), d, true);
        p[kb * 4 + q] = d;
      }
  };
  // O^T += V^T P^T, the products times 2^(E-64) (E8M0 scale ebits of the B
  // operand: for output column j it is read from lanes j and j+32, both this
  // query's), and the row sum += 2^(E-64) 1^T P^T
  auto pv = [&](const uint8_t *sv, const i32x8 &p, int ebits) {
    const f32x4 lt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, p, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                      0x7F7F7F7F, 0, 0x7F7F7F7F);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 lo = *reinterpret_cast<const uint4 *>(sv + t * 32 * KT8 + voff[0]);
      const uint4 hi = *reinterpret_cast<const uint4 *>(sv + t * 32 * KT8 + voff[1]);
      i32x8 va;
      va[0] = lo.x; va[1] = lo.y; va[2] = lo.z; va[3] = lo.w;
      va[4] = hi.x; va[5] = hi.y; va[6] = hi.z; va[7] = hi.w;
      o[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, p, o[t], 0, 0, 0, 0x7F7F7F7F, 0, ebits);
    }
    lsum = fmaf(lt[0], __int_as_float((ebits & 0xFF) << 23), lsum);   // 2^(byte - 127)
  };

  constexpr std::integral_constant<int, 0> P0{};
  constexpr std::integral_constant<int, 1> P1{};
  const bool ragged_last = (Lk % KT8) != 0;

  gloadK(0, P0);
  if (ntiles > 1) gloadK(1, P1);
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  i32x16 sa[2], sb[2];
  qk(sK0, sa);
  float m;   // running max, log2 units, minus XTOP8
  int E = 0;  // its rise since the first tile (whole log2 units)
  {
    float x[2][16];
    const float c = cq * ksp[0];
    expo(sa, c, -K0F * c, ntiles == 1 && ragged_last, 0, x);
    const float lm = lanemax(x);
    m = fmaxf(lm, half_swap(lm)) - XTOP8;
  }
  __syncthreads();   // every wavefront has read K(0)

  // iteration j: LDS holds K(j+1) and V(j-1) in stage (j+1)&1; the scores of
  // tile j are in scur, the probabilities of tile j-1 in pprev.  has_next: tile
  // j+1 exists; load_k2: tile j+2 exists; do_pv: j >= 1; ragged: tile j is
  // the last, ragged tile.
  auto step = [&](auto P, int j, const i32x16 (&scur)[2], i32x16 (&snxt)[2], i32x8 &pcur,
                  const i32x8 &pprev, int &ecur, int eprev, bool has_next, bool load_k2, bool do_pv,
                  bool ragged) {
    const auto Q = other(P);
    if (load_k2) gloadK(j + 2, P);      // stage of K(j), read in iteration j-1
    gloadV(j, P);                        // stage of V(j-2), read in iteration j-1
    const float c = cq * ksp[j];
    // region 1 -- matrix unit: PV of tile j-1; vector unit: the lane max of
    // tile j's biased scores (as floats 1.5 * 2^23 + S, ordered like S)
    if (do_pv) pv(vbuf(Q), pprev, eprev);
    const float lx = fmaf(rawmax(scur, ragged, j), c, -fmaf(K0F, c, m));
    if (do_pv) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // V fragments of the first two MFMAs
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // the fragment two MFMAs ahead
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);   // 4 VALU
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
      }
    }
    if (__builtin_amdgcn_ballot_w64(lx > XMAX8) != 0) {
      // raise the running max by whole log2 units, so that this tile's
      // largest probability lands in (2^6, 2^7]
      const float dm = ceilf(fmaxf(fmaxf(lx, half_swap(lx)) - XTOP8, 0.f));
      m += dm;
      E += (int)dm;
      if (E > 150) {
        // the terms accumulated so far are below 2^-130 of the new ones
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int t = 0; t < 4; ++t) o[t][r] = 0.f;
        lsum = 0.f;
        E = 0;
      }
    }
    ecur = (63 + E) * 0x01010101;   // E8M0 of 2^(E-64) in every byte: this tile's scale
    // region 2 -- matrix unit: the scores of tile j+1; vector unit: the
    // exponents and probabilities of tile j
    if (has_next) qk(kbuf(Q), snxt);
    float x[2][16];
    expo(scur, c, -fmaf(K0F, c, m), ragged, j, x);
    probs(x, pcur);
    if (has_next) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // K fragments of the first two MFMAs
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the fragment two MFMAs ahead
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // 6 VALU (FMA, E4M3 packing)
        __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);   // 4 exponentials
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // K(j+2), V(j) landed; LDS reads done
    __syncthreads();
  };

  i32x8 pa, pb;
  int ea = 63 * 0x01010101, eb = 63 * 0x01010101;
#pragma unroll
  for (int r = 0; r < 8; ++r) pa[r] = pb[r] = 0;
  step(P0, 0, sa, sb, pa, pb, ea, eb, ntiles > 1, ntiles > 2, false, ntiles == 1 && ragged_last);
  int j = 1;
  for (; j + 3 < ntiles; j += 2) {
    step(P1, j, sb, sa, pb, pa, eb, ea, true, true, true, false);
    step(P0, j + 1, sa, sb, pa, pb, ea, eb, true, true, true, false);
  }
  // the last tiles with run-time stages; scores of tile j in sb, P(j-1) in pa
  for (; j < ntiles; ++j) {
    step(j & 1, j, sb, sa, pb, pa, eb, ea, j + 1 < ntiles, j + 2 < ntiles, true,
         j == ntiles - 1 && ragged_last);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sb[kb] = sa[kb];
    pa = pb;
    ea = eb;
  }
  pv(vbuf((ntiles - 1) & 1), pa, ea);
  // the MFMAs read operands across the whole wavefront: keep the last ones
  // (and their LDS reads) out of the row-guarded store below, where the
  // compiler would otherwise sink them under a partial EXEC mask
  asm volatile("" ::"v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(lsum));

  // ---- normalise, undo the V channel scales, store: lane holds
  // O^T[hd = t*32 + (r/4)*8 + g*4 + r%4][query qrow]
  if (!qok) return;
  const float inv = 1.0f / lsum;
  const float *vsp = a.vs + (long)b * (H * HD8) + h * HD8;
  const long orow = (long)(b * Lq + qrow);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int hd0 = t * 32 + rb * 8 + g * 4;
      const float4 sv = *reinterpret_cast<const float4 *>(vsp + hd0);
      bf16x4 ov;
      ov[0] = f2bf(o[t][rb * 4 + 0] * sv.x * inv);
      ov[1] = f2bf(o[t][rb * 4 + 1] * sv.y * inv);
      ov[2] = f2bf(o[t][rb * 4 + 2] * sv.z * inv);
      ov[3] = f2bf(o[t][rb * 4 + 3] * sv.w * inv);
      *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(a.o) + orow * a.ldo + h * HD8 + hd0) = ov;
    }
}

}  // namespace

hipError_t launch_quant_attn8(const Attn8Quant &z, hipStream_t s) {
  if (z.B <= 0 || z.H <= 0 || z.Lq <= 0 || z.Lk <= 0) return hipSuccess;
  const long qgroups = (long)z.B * z.Lq * z.H;
  k_quant_q8<<<(int)((qgroups + 15) / 16), 256, 0, s>>>(reinterpret_cast<const bf16 *>(z.q), z.ldq, z.B * z.Lq, z.H,
                                                         reinterpret_cast<int8_t *>(z.q8), z.ldq8, z.qs);
  const int nkb = (z.Lk + KT8 - 1) / KT8;
  k_quant_k8<<<z.B * z.H * nkb, 256, 0, s>>>(reinterpret_cast<const bf16 *>(z.k), z.ldk, z.B, z.H, z.Lk,
                                             reinterpret_cast<int8_t *>(z.k8), z.ldk8, z.ks);
  k_quant_vt8<<<z.B * z.H * HD8, 256, 0, s>>>(reinterpret_cast<const bf16 *>(z.vt), z.ldv, z.vt_bstride, z.H, z.Lk,
                                              reinterpret_cast<uint8_t *>(z.v8t), z.ldv8, z.v8_bstride, z.vs);
  return hipGetLastError();
}

hipError_t launch_attention8(const Attn8Desc &a, hipStream_t s) {
  if (a.B <= 0 || a.H <= 0 || a.Lq <= 0 || a.Lk <= 0) return hipSuccess;
  const int nqt = (a.Lq + QW8 - 1) / QW8;
  k_attn_i8f8<<<a.B * a.H * nqt, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace wan
