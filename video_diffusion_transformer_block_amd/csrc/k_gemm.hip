// GEMMs of the DiT block: C[M,N] = A[M,K] . B[N,K]^T (+ bias) with fused
// epilogues (bf16 store, float32 store, tanh-GELU, gated residual add into
// the float32 stream).  These are the block's Linear layers: QKV, the
// attention out-projections, the cross-attention Q/K/V projections, the FFN
// ("Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)",
// table 配置表 for the widths), patchify as a GEMM over gathered patches.
//
// bf16 path: 256x256x64 block tile, 8 wavefronts (two per SIMD) in a 2x4
// grid, each owning a 128x64 tile of 4x2 v_mfma_f32_32x32x16_bf16
// accumulators.  A and B tiles go global -> LDS directly
// (buffer_load_dwordx4 ... lds) into a 16-byte-chunk XOR swizzle that keeps the
// 16 lanes one ds_read_b128 cycle serves on distinct banks.  The K loop is
// software-pipelined: the LDS reads of the next k-substep are interleaved
// with the MFMAs of the current one, and the last substep's MFMAs run across
// the stage switch while the next stage's first fragments and the loads two
// K tiles ahead are issued (two LDS stages, one barrier per K tile).  Tail rows / columns
// load a clamped (in-bounds) row and are never stored.  Tiles are visited in
// groups of 8 M-tiles so that the 32 workgroups an XCD runs at once share A
// and B slices in that XCD's L2.  The MFMAs compute the tile transposed
// (operands swapped), so each lane holds runs of 4 consecutive columns of one
// output row; both epilogues stage a wavefront's slab through LDS and store
// whole row segments.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 256, GBN = 256;
constexpr int GBK = 64, NSTAGE = 2;     // K tile 64 (four MFMA k-substeps), two LDS stages
constexpr int GW = 8;            // wavefronts per workgroup (two per SIMD)
constexpr int GROUP_M = 8;       // M-tiles per L2 group

// 16-byte chunk XOR swizzle of a tile row of CH chunks: the 16 rows one
// ds_read_b128 cycle touches land on distinct (256-byte-period) bank groups
template <int CH> WAN_DEV int swz_row(int row);
template <> WAN_DEV int swz_row<8>(int row) { return (row >> 1) & 7; }   // 128-byte rows
template <> WAN_DEV int swz_row<4>(int row) { return (row >> 2) & 3; }   // 64-byte rows

typedef __attribute__((address_space(3))) void *lds_ptr;

// s_waitcnt vmcnt(N) lgkmcnt(0), N <= 15: direct loads older than the last N
// have landed and every LDS read of this wavefront has returned
template <int N> WAN_DEV void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0070 | N); }

// Epilogue of bf16 outputs through LDS: per wave 4 slabs of 32 rows x 64
// columns (fp32, padded rows), written from the transposed tile's runs of 4
// columns, read back so that every lane finishes 8 contiguous columns of one
// row per pass and stores 16 bytes.  Everything it reads
// from global memory (bias, FP8 scales) is loaded before its first store: the
// memory counter retires in issue order, so a load issued after a store would
// wait for that store.  The caller has synchronised the workgroup.
template <int KIND, bool BROWS, bool SCALED>
WAN_DEV void epilogue(const GemmDesc &g, const f32x16 (&acc)[4][2], float *lds, int w, int lane,
                      int m0, int n0, int wm, int wn) {
  static_assert(KIND == OUT_BF16 || KIND == OUT_GELU, "bf16 outputs only");
  const int half = lane >> 5, l32 = lane & 31;
  constexpr int EP = 68;
  float *ep = lds + w * 32 * EP;
  // read-back: in pass p a lane finishes row 8p + lane/8 of the slab, columns
  // c8 .. c8+7 (c8 = 8 (lane % 8)), so one store instruction writes 8 rows of
  // 128 contiguous bytes (the previous mapping, 2 lanes per row 32 columns
  // apart, spread each store over 32 rows and ran 3-8% slower)
  const int rr = lane >> 3, c8 = (lane & 7) * 8;
  const int n = n0 + wn * 64 + c8;             // this lane's first column
  const int mb = m0 + wm * 128 + rr;           // row of slab 0, pass 0
  const bf16 *bias = reinterpret_cast<const bf16 *>(g.bias);
  constexpr bool CADD = !BROWS, CMUL = SCALED && BROWS;
  // column terms of the lane's 8 columns, row terms of its 16 rows (indices
  // clamped into the matrix; clamped values are never stored), all loaded
  // before the first store
  bf16x8 cadd;
  float cmul[8], radd[16], rmul[16];
  if (CADD && bias && n + 8 <= g.N) {
    const uint4 u = ld16(bias + n);
    cadd = *reinterpret_cast<const bf16x8 *>(&u);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) cadd[k] = CADD && bias ? bias[n + k < g.N ? n + k : g.N - 1] : (bf16)0.f;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    cmul[k] = CMUL ? g.b_scale[g.b_per_col ? (n + k < g.N ? n + k : g.N - 1) : 0] : 1.f;
  const float csc = SCALED && !CMUL ? g.b_scale[0] : 1.f;   // a per-tensor column scale
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mc = min(mb + (i >> 2) * 32 + (i & 3) * 8, g.M - 1);
    radd[i] = bias && BROWS ? (float)bias[mc] : 0.f;
    rmul[i] = SCALED ? g.a_scale[g.a_per_row ? mc : 0] * csc : 1.f;
  }
  const int lim = g.npad > g.N ? g.npad : g.N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the transposed tile: lane l holds row l%32, columns 8q + 4(l/32) .. +3
    // of each 32-column block jj -- one 16-byte LDS write per run
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(ep + l32 * EP + jj * 32 + q * 8 + half * 4) =
            make_float4(acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3]);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 8 * p + rr;
      const int m = mb + i * 32 + 8 * p;
      if (m < g.M && n < lim) {
        const float4 u0 = *reinterpret_cast<const float4 *>(ep + r * EP + c8);
        const float4 u1 = *reinterpret_cast<const float4 *>(ep + r * EP + c8 + 4);
        float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        const int ri = i * 4 + p;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[k] = v[k] * rmul[ri] * (CMUL ? cmul[k] : 1.f) + radd[ri] + (CADD ? (float)cadd[k] : 0.f);
          if (KIND == OUT_GELU) v[k] = gelu_tanh(v[k]);
          if (KIND == OUT_BF16 && n < g.scale_cols) v[k] *= g.col_scale;
        }
        bf16 *c = reinterpret_cast<bf16 *>(g.C) + (long)m * g.ldc + n;
        if (n + 8 <= g.N) {
          bf16x8 o;
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = f2bf(v[k]);
          // non-temporal: the output stream does not allocate in L2 over the
          // operand tiles (block step 8.11 -> 8.04 ms; the same hint on the
          // float32 stream measured no gain)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&o), reinterpret_cast<u32x4 *>(c));
        } else {
          for (int k = 0; k < 8 && n + k < lim; ++k) c[k] = n + k < g.N ? f2bf(v[k]) : f2bf(0.f);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
}

// Epilogue of float32 outputs through LDS: the slabs of the bf16 epilogue,
// read back with 16 lanes per row (4 columns, 16 bytes each), so one store
// writes 4 rows of 256 contiguous bytes.  The gated residual reads x[m, n]
// with the same pattern; the gate rows of the wave's 128 rows are loaded
// before the first store when those rows span at most two batch samples.
template <int KIND, bool SCALED>
WAN_DEV void epilogue_f32(const GemmDesc &g, const f32x16 (&acc)[4][2], float *lds, int w, int lane,
                          int m0, int n0, int wm, int wn) {
  static_assert(KIND == OUT_F32 || KIND == OUT_RESID, "float32 outputs only");
  const int half = lane >> 5, l32 = lane & 31;
  constexpr int EP = 68;
  float *ep = lds + w * 32 * EP;
  const int rr = lane >> 4, c4 = (lane & 15) * 4;
  const int n = n0 + wn * 64 + c4;
  const int mw = m0 + wm * 128;
  const bool full = n + 4 <= g.N;
  const bf16 *bias = reinterpret_cast<const bf16 *>(g.bias);
  float b4[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias && n < g.N) {
    if (full) {
      const uint2 u = *reinterpret_cast<const uint2 *>(bias + n);
      const bf16 *e = reinterpret_cast<const bf16 *>(&u);
#pragma unroll
      for (int k = 0; k < 4; ++k) b4[k] = (float)e[k];
    } else {
      for (int k = 0; k < 4; ++k) b4[k] = n + k < g.N ? (float)bias[n + k] : 0.f;
    }
  }
  float rmul[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mc = min(mw + i * 32 + l32, g.M - 1);
    rmul[i] = SCALED ? g.a_scale[g.a_per_row ? mc : 0] * g.b_scale[0] : 1.f;
  }
  // gates of the first and the last row's sample (columns clamped into N)
  float4 gA = make_float4(1.f, 1.f, 1.f, 1.f), gB = gA;
  int mB = 0x7fffffff;          // first row of the second sample
  bool two = true;
  if (KIND == OUT_RESID && g.gate) {
    const int rpb = g.rows_per_batch;
    const int bA = mw / rpb, bL = min(mw + 127, g.M - 1) / rpb;
    two = bL - bA <= 1;
    mB = (bA + 1) * rpb;
    const int nc = full ? n : 0;
    const float *gp = g.gate + nc;
    gA = *reinterpret_cast<const float4 *>(gp + (long)bA * g.gate_bstride);
    gB = *reinterpret_cast<const float4 *>(gp + (long)bL * g.gate_bstride);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(ep + l32 * EP + jj * 32 + q * 8 + half * 4) =
            make_float4(acc[i][jj][4 * q] * rmul[i], acc[i][jj][4 * q + 1] * rmul[i],
                        acc[i][jj][4 * q + 2] * rmul[i], acc[i][jj][4 * q + 3] * rmul[i]);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    float4 xv[8];
    if (KIND == OUT_RESID && full) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int m = mw + i * 32 + 4 * p + rr;
        if (m < g.M) xv[p] = *reinterpret_cast<const float4 *>(g.X + (long)m * g.ldx + n);
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = 4 * p + rr;
      const int m = mw + i * 32 + r;
      if (m < g.M && n < g.N) {
        const float4 u = *reinterpret_cast<const float4 *>(ep + r * EP + c4);
        float v[4] = {u.x + b4[0], u.y + b4[1], u.z + b4[2], u.w + b4[3]};
        if (KIND == OUT_F32) {
          float *c = reinterpret_cast<float *>(g.C) + (long)m * g.ldc + n;
          if (full) *reinterpret_cast<float4 *>(c) = make_float4(v[0], v[1], v[2], v[3]);
          else
            for (int k = 0; k < 4 && n + k < g.N; ++k) c[k] = v[k];
        } else {
          float gg[4] = {1.f, 1.f, 1.f, 1.f};
          if (g.gate) {
            if (two && full) {
              const float4 s = m < mB ? gA : gB;
              gg[0] = s.x; gg[1] = s.y; gg[2] = s.z; gg[3] = s.w;
            } else {
              const float *gp = g.gate + (long)(m / g.rows_per_batch) * g.gate_bstride + n;
              for (int k = 0; k < 4; ++k) gg[k] = n + k < g.N ? gp[k] : 0.f;
            }
          }
          float *xp = g.X + (long)m * g.ldx + n;
          if (full) {
            float4 x = xv[p];
            x.x += gg[0] * v[0]; x.y += gg[1] * v[1]; x.z += gg[2] * v[2]; x.w += gg[3] * v[3];
            *reinterpret_cast<float4 *>(xp) = x;
          } else {
            for (int k = 0; k < 4 && n + k < g.N; ++k) xp[k] += gg[k] * v[k];
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
}

// Every tile is computed transposed (C^T = B A^T: MFMA operands swapped), so
// a lane holds runs of 4 consecutive columns of one output row.  Both
// epilogues stage a wave's 32-row slab through LDS (one 16-byte write per run)
// and read it back row-contiguous, so that each store instruction covers a few
// whole 128-256 byte row segments (2 lanes per row, 32 columns apart, wrote
// 32 rows x 32 bytes per float32 store and ran 12% slower at d x d).
template <int KIND> constexpr bool epi_f32() { return KIND == OUT_F32 || KIND == OUT_RESID; }

template <int KIND, bool BROWS>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(GemmDesc g) {
  constexpr int CH = GBK / 8;                 // 16-byte chunks per tile row
  constexpr int RPB = 1024 / (GBK * 2);       // rows per 1-KB direct-load block
  constexpr int BPW = GBM / RPB / GW;         // blocks per wavefront per operand tile
  constexpr int KS = GBK / 16;                // MFMA k-substeps per K tile
  constexpr int LPT = 2 * BPW;                // direct loads per wavefront per K tile
  __shared__ __attribute__((aligned(16))) bf16 smem[NSTAGE * (GBM + GBN) * GBK];
  bf16 *sA = smem;                            // [stage][256][GBK]
  bf16 *sB = smem + NSTAGE * GBM * GBK;       // [stage][256][GBK]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int half = lane >> 5, l32 = lane & 31;
  const int tiles_m = (g.M + GBM - 1) / GBM;
  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int group = GROUP_M * tiles_n;
  const int first_m = (bid / group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (bid % group) % gm;
  const int tn = (bid % group) / gm;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const bf16 *A = reinterpret_cast<const bf16 *>(g.A);
  const bf16 *Bm = reinterpret_cast<const bf16 *>(g.B);

  // global -> LDS, direct (buffer_load_dwordx4 ... lds): wavefront w fills the
  // 1-KB blocks w*BPW .. of each tile; lane i lands at block base + 16 i =
  // row blk*RPB + i/CH, physical chunk i%CH, so it fetches the logical chunk
  // (i%CH) ^ swz(row) of that row.
  // buffer descriptors over A and B (byte sizes < 4 GiB, checked on the host);
  // per-lane byte offsets of the (clamped, so always in-range) rows
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)A, 0, (int)((unsigned)g.M * (unsigned)g.lda * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)Bm, 0, (int)((unsigned)g.N * (unsigned)g.ldb * 2u), 0x00020000);
  int oa[BPW], ob[BPW];
#pragma unroll
  for (int r = 0; r < BPW; ++r) {
    const int row = (w * BPW + r) * RPB + lane / CH;
    const int c = (lane % CH) ^ swz_row<CH>(row);
    oa[r] = (int)(((unsigned)min(m0 + row, g.M - 1) * (unsigned)g.lda + c * 8) * 2u);
    ob[r] = (int)(((unsigned)min(n0 + row, g.N - 1) * (unsigned)g.ldb + c * 8) * 2u);
  }
  auto gload = [&](int kt, int st) {
    const int k0b = kt * GBK * 2;      // byte offset of the K tile (scalar)
    bf16 *da = sA + st * GBM * GBK + w * BPW * 512;
    bf16 *db = sB + st * GBN * GBK + w * BPW * 512;
#pragma unroll
    for (int r = 0; r < BPW; ++r) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(da + r * 512), 16, oa[r], k0b, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(db + r * 512), 16, ob[r], k0b, 0, 0);
    }
  };

  // fragment offsets (elements) for k-substep ks: chunk ks*2 + half; the
  // row swizzle only depends on l32 (row offsets are multiples of 32)
  int aoff[KS], boff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    aoff[ks] = (wm * 128 + l32) * GBK + (((ks * 2 + half) ^ swz_row<CH>(l32)) * 8);
    boff[ks] = (wn * 64 + l32) * GBK + (((ks * 2 + half) ^ swz_row<CH>(l32)) * 8);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment registers: three slots, so the LDS reads of substep u+2 are in
  // flight while substep u is multiplied (slot of substep u = u mod 3)
  bf16x8 fa[3][4], fb[3][2];
  auto frags = [&](int st, int ks, int slot) {
    const bf16 *a_s = sA + st * GBM * GBK;
    const bf16 *b_s = sB + st * GBN * GBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8 *>(a_s + aoff[ks] + i * 32 * GBK);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8 *>(b_s + boff[ks] + j * 32 * GBK);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);
  };
  // scheduling hint: one MFMA, one LDS read, alternately (6 reads), then 2 MFMAs
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  const int KT = g.K / GBK;
  // prologue: tiles 0 .. NSTAGE-1 in flight (one per stage); wait for tile 0
#pragma unroll
  for (int p = 0; p < NSTAGE; ++p)
    if (p < KT) gload(p, p);
  if (KT >= NSTAGE) wait_vm<(NSTAGE - 1) * LPT>();
  else wait_vm<0>();
  __syncthreads();
  frags(0, 0, 0);
  frags(0, 1, 1);

  // One K tile (KS == 4 substeps); `sb` = slot of its substep 0 (= kt mod 3).
  // Substeps 0, 1 read the stage's substeps 2, 3; then, once every read of
  // this stage is issued, the barrier; substeps 2, 3 read the next stage's
  // substeps 0, 1 and the freed stage receives tile kt + NSTAGE.
  auto tile = [&](int kt, int sb) {
    const int st = kt % NSTAGE, nst = (kt + 1) % NSTAGE;
    frags(st, 2, (sb + 2) % 3);
    mfmas(sb);
    interleave();
    frags(st, 3, sb);          // slot of substep 3 == slot of substep 0 (its MFMAs are issued)
    mfmas((sb + 1) % 3);
    interleave();
    if (kt + NSTAGE - 1 <= KT - 1) wait_vm<(NSTAGE - 2) * LPT>();
    else wait_vm<0>();
    __syncthreads();
    if (kt + NSTAGE < KT) gload(kt + NSTAGE, st);
    // next stage's substeps 0, 1 (on the last tile a harmless, unused read)
    frags(nst, 0, (sb + 1) % 3);
    mfmas((sb + 2) % 3);
    interleave();
    frags(nst, 1, (sb + 2) % 3);
    mfmas(sb);
    interleave();
  };
  int kt = 0;
  for (; kt + 3 <= KT; kt += 3) {   // three tiles: 12 substeps, slots cycle back to 0
    tile(kt, 0);
    tile(kt + 1, 1);
    tile(kt + 2, 2);
  }
  if (kt < KT) tile(kt, 0);
  if (kt + 1 < KT) tile(kt + 1, 1);

  __syncthreads();
  if constexpr (epi_f32<KIND>()) {
    epilogue_f32<KIND, false>(g, acc, reinterpret_cast<float *>(smem), w, lane, m0, n0, wm, wn);
  } else {
    epilogue<KIND, BROWS, false>(g, acc, reinterpret_cast<float *>(smem), w, lane, m0, n0, wm, wn);
  }
}

// FP8 operands (OCP E4M3; "Wan: Open and Advanced Large-Scale Video Generative
// Models (Wan 2.1)", section Infra / 推理优化: FP8 GEMM with per-tensor weight
// and per-token activation scales).  256x256 output tile, 8 wavefronts (2x4,
// 128x64 each), v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales (E8M0
// 127).  A K tile is 64 one-byte elements (one MFMA depth): 64-byte rows,
// 16-byte chunks XOR-swizzled by (row >> 2) & 3, two LDS stages of 32 KB, so
// every fragment read fits the LDS immediate offset.  A fragment is 32 bytes
// per lane -- row l%32, k = 32*(l/32) .. +32, two ds_read_b128 -- with A and B
// in the same k order, which is all the dot product needs.  Per tile: the
// loads of tile kt+2 start, the 8 MFMAs of tile kt run from registers, one
// barrier, then the fragments of tile kt+1 are read into the same registers
// while those MFMAs execute.  The epilogues (LDS-staged, as for bf16
// operands) scale by the row scale times the column scale.  This kernel takes the
// shapes whose K is not a multiple of 256; k_gemm_fp8w below the rest.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int KIND, bool BROWS>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8(GemmDesc g) {
  constexpr int GBK8 = 64;                    // K tile, bytes = elements
  constexpr int RPB = 1024 / GBK8;            // rows per 1-KB direct-load block (16)
  constexpr int BPW = GBM / RPB / GW;         // blocks per wavefront per operand tile (2)
  constexpr int LPT = 2 * BPW;                // direct loads per wavefront per K tile
  // one LDS variable per stage and operand (16 KB each): the compiler gives
  // each its own alias scope, so reads of one stage need not wait for the
  // direct loads still landing in the other; stages are picked with
  // compile-time parities in the steady-state loop
  __shared__ __attribute__((aligned(16))) uint8_t sA0[GBM * GBK8];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[GBM * GBK8];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[GBN * GBK8];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[GBN * GBK8];
  auto abuf = [&](auto P) -> uint8_t * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sA1 : sA0;
    else if constexpr (decltype(P)::value == 0) return sA0;
    else return sA1;
  };
  auto bbuf = [&](auto P) -> uint8_t * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sB1 : sB0;
    else if constexpr (decltype(P)::value == 0) return sB0;
    else return sB1;
  };
  auto other = [](auto P) {
    if constexpr (std::is_integral_v<decltype(P)>) return 1 - P;
    else return std::integral_constant<int, 1 - decltype(P)::value>{};
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // a workgroup barrier without a memory fence: a fence would wait for every
  // direct load in flight; the counter waits before it order the hardware and
  // the empty asm statements keep the compiler from moving memory accesses
  auto barrier = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int half = lane >> 5, l32 = lane & 31;
  const int tiles_m = (g.M + GBM - 1) / GBM;
  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int group = GROUP_M * tiles_n;
  const int first_m = (bid / group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (bid % group) % gm;
  const int tn = (bid % group) / gm;
  const int m0 = tm * GBM, n0 = tn * GBN;

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.A, 0, (int)((unsigned)g.M * (unsigned)g.lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.B, 0, (int)((unsigned)g.N * (unsigned)g.ldb), 0x00020000);
  int oa[BPW], ob[BPW];
#pragma unroll
  for (int r = 0; r < BPW; ++r) {
    const int row = (w * BPW + r) * RPB + lane / 4;
    const int c = (lane % 4) ^ swz_row<4>(row);
    oa[r] = (int)((unsigned)min(m0 + row, g.M - 1) * (unsigned)g.lda + c * 16);
    ob[r] = (int)((unsigned)min(n0 + row, g.N - 1) * (unsigned)g.ldb + c * 16);
  }
  auto gload = [&](int kt, auto st) {
    const int k0b = kt * GBK8;
    uint8_t *da = abuf(st) + w * BPW * 1024;
    uint8_t *db = bbuf(st) + w * BPW * 1024;
#pragma unroll
    for (int r = 0; r < BPW; ++r) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(da + r * 1024), 16, oa[r], k0b, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(db + r * 1024), 16, ob[r], k0b, 0, 0);
    }
  };
  // byte offsets of a fragment's two chunks (logical 2 half + {0, 1}); the row
  // swizzle depends only on l32 (row offsets are multiples of 32)
  int aoff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = ((2 * half + j) ^ swz_row<4>(l32)) * 16;
    aoff[j] = (wm * 128 + l32) * GBK8 + c;
    boff[j] = (wn * 64 + l32) * GBK8 + c;
  }

  // accumulators in AGPRs (an AGPR operand makes the compiler split the 256
  // registers 128 / 128); fragments and addresses use the VGPRs
  asm volatile("; accumulators in AGPRs" :: "a"(0.0f));
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  i32x8 fa[4], fb[2];
  auto frag = [&](const uint8_t *p, const int (&off)[2]) -> i32x8 {
    const uint4 lo = *reinterpret_cast<const uint4 *>(p + off[0]);
    const uint4 hi = *reinterpret_cast<const uint4 *>(p + off[1]);
    i32x8 v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  auto frags = [&](auto st) {
    const uint8_t *a_s = abuf(st), *b_s = bbuf(st);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag(a_s + i * 32 * GBK8, aoff);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = frag(b_s + j * 32 * GBK8, boff);
  };
  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0,
                                                                    0x7F7F7F7F, 0, 0x7F7F7F7F);
  };

  const int KT = g.K / GBK8;
  gload(0, I0{});
  if (KT > 1) gload(1, I1{});
  if (KT > 1) wait_vm<LPT>();
  else wait_vm<0>();
  barrier();
  frags(I0{});
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): tile 0's fragments are in registers
  barrier();                            // every wavefront has read stage 0

  // tile kt (fragments in registers, stage kt&1 free, stage (kt+1)&1 holding
  // tile kt+1 or still receiving it): start the loads of tile kt+2 into the
  // free stage (load2), issue the MFMAs, wait for tile kt+1, one barrier, read
  // its fragments (next) while the MFMAs execute, and a second barrier so the
  // stage just read may be refilled by the next tile.
  auto tile = [&](int kt, auto st, bool load2, bool next) {
    if (load2) gload(kt + 2, st);
    mfmas();
    __builtin_amdgcn_sched_barrier(0);
    if (load2) wait_vm<LPT>();
    else wait_vm<0>();
    barrier();
    if (next) frags(other(st));
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): fragments read
    barrier();
  };
  int kt = 0;
  for (; kt + 3 < KT; kt += 2) {   // tiles kt .. kt+3 exist
    tile(kt, I0{}, true, true);
    tile(kt + 1, I1{}, true, true);
  }
  for (; kt < KT; ++kt)             // the last 1 .. 3 tiles: one generic copy with run-time flags
    tile(kt, kt & 1, kt + 2 < KT, kt + 1 < KT);

  // 8 wavefronts x 32 rows x 68 floats staged through an LDS buffer of its own
  __shared__ __attribute__((aligned(16))) float sEp[GW * 32 * 68];
  if constexpr (epi_f32<KIND>()) {
    static_assert(!BROWS, "bias along rows: bf16 outputs only");
    epilogue_f32<KIND, true>(g, acc, sEp, w, lane, m0, n0, wm, wn);
  } else {
    epilogue<KIND, BROWS, true>(g, acc, sEp, w, lane, m0, n0, wm, wn);
  }
}

// FP8 operands with K a multiple of 256 (every Linear layer of the models:
// K = 1536, 5120, 8960, 13824): the same output tile, wavefronts and MFMA,
// with 128-deep K tiles -- the bf16 kernel's 128-byte rows, swizzle and
// direct loads -- so one barrier and one load wait cover 16 MFMAs per
// wavefront instead of 8.  A tile is two k-substeps of 64.  The fragments sit
// in one set of registers that is refilled as it frees up (see `sub`), so
// each LDS read runs three or more MFMAs ahead of its use and two stages of
// 64 KB fit beside it.  The accumulation order over K is the 64-deep kernel's,
// so the two give bitwise equal outputs.
template <int KIND, bool BROWS>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8w(GemmDesc g) {
  constexpr int GBK8 = 128;                   // K tile, bytes = elements: 128-byte rows, as the bf16 kernel's
  constexpr int CH = GBK8 / 16;               // 16-byte chunks per tile row (8)
  constexpr int RPB = 1024 / GBK8;            // rows per 1-KB direct-load block (8)
  constexpr int BPW = GBM / RPB / GW;         // blocks per wavefront per operand tile (4)
  constexpr int LPT = 2 * BPW;                // direct loads per wavefront per K tile
  constexpr int SB = (GBM + GBN) * GBK8;      // bytes per stage: A rows, then B rows
  // one LDS variable per stage (the compiler gives each its own alias scope,
  // so reads of one stage need not wait for direct loads landing in the other)
  __shared__ __attribute__((aligned(16))) uint8_t s0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t s1[SB];
  auto stage = [&](auto ST) -> uint8_t * {
    if constexpr (decltype(ST)::value == 0) return s0;
    else return s1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using TA = std::true_type;
  using FA = std::false_type;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int half = lane >> 5, l32 = lane & 31;
  const int tiles_m = (g.M + GBM - 1) / GBM;
  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int group = GROUP_M * tiles_n;
  const int first_m = (bid / group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (bid % group) % gm;
  const int tn = (bid % group) / gm;
  const int m0 = tm * GBM, n0 = tn * GBN;

  // global -> LDS as in the bf16 kernel: lane i of a 1-KB block lands at row
  // blk*RPB + i/CH, physical chunk i%CH, and fetches logical chunk (i%CH) ^ swz(row)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.A, 0, (int)((unsigned)g.M * (unsigned)g.lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.B, 0, (int)((unsigned)g.N * (unsigned)g.ldb), 0x00020000);
  int oa[BPW], ob[BPW];
#pragma unroll
  for (int r = 0; r < BPW; ++r) {
    const int row = (w * BPW + r) * RPB + lane / CH;
    const int c = (lane % CH) ^ swz_row<CH>(row);
    oa[r] = (int)((unsigned)min(m0 + row, g.M - 1) * (unsigned)g.lda + c * 16);
    ob[r] = (int)((unsigned)min(n0 + row, g.N - 1) * (unsigned)g.ldb + c * 16);
  }
  auto gload = [&](int kt, auto st) {
    const int k0b = kt * GBK8;
    uint8_t *da = stage(st) + w * BPW * 1024;
    uint8_t *db = stage(st) + GBM * GBK8 + w * BPW * 1024;
#pragma unroll
    for (int r = 0; r < BPW; ++r) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(da + r * 1024), 16, oa[r], k0b, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(db + r * 1024), 16, ob[r], k0b, 0, 0);
    }
  };
  // k-substep ks (64 bytes of K): a lane's fragment is 32 bytes, logical
  // chunks 4 ks + 2 half + {0, 1} of its row; the swizzle depends only on l32
  int aoff[2][2], boff[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = ((4 * ks + 2 * half + j) ^ swz_row<CH>(l32)) * 16;
      aoff[ks][j] = (wm * 128 + l32) * GBK8 + c;
      boff[ks][j] = GBM * GBK8 + (wn * 64 + l32) * GBK8 + c;
    }

  // accumulators in AGPRs (an AGPR operand makes the compiler split the 256
  // registers 128 / 128); fragments and addresses use the VGPRs
  asm volatile("; accumulators in AGPRs" :: "a"(0.0f));
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // one set of fragment registers, refilled as they free up: the MFMAs of a
  // substep run in one of two orders, and after each MFMA that was the last
  // user of a fragment, that fragment of the next substep is read into it.
  // Order A: (0,0) (1,0) (2,0) (3,0) (3,1) (2,1) (1,1) (0,1); order B: (3,0)
  // (2,0) (1,0) (0,0) (0,1) (1,1) (2,1) (3,1) (A fragment, B fragment).  Each
  // order consumes the fragments in the order the other one frees them, so
  // every read runs at least three MFMAs ahead of its use.
  i32x8 fa[4], fb[2];
  auto frag = [&](const uint8_t *p, const int (&off)[2]) -> i32x8 {
    const uint4 lo = *reinterpret_cast<const uint4 *>(p + off[0]);
    const uint4 hi = *reinterpret_cast<const uint4 *>(p + off[1]);
    i32x8 v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  auto sub = [&](auto ORDER_A, auto READS, const uint8_t *rs, auto RKS) __attribute__((always_inline)) {
    constexpr int rks = decltype(RKS)::value;
    constexpr bool oa_ = decltype(ORDER_A)::value, rd = decltype(READS)::value;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int j = n >> 2;
      const int i = oa_ ? (j ? 7 - n : n) : (j ? n - 4 : 3 - n);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0,
                                                                  0x7F7F7F7F, 0, 0x7F7F7F7F);
      if constexpr (rd) {
        if (n == 3) fb[0] = frag(rs, boff[rks]);
        if (n >= 4) fa[i] = frag(rs + i * 32 * GBK8, aoff[rks]);
        if (n == 7) fb[1] = frag(rs + 32 * GBK8, boff[rks]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int KT = g.K / GBK8;                  // even (K % 256 == 0, checked on the host)
  gload(0, I0{});
  gload(1, I1{});
  wait_vm<LPT>();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = frag(s0 + i * 32 * GBK8, aoff[0]);
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[j] = frag(s0 + j * 32 * GBK8, boff[0]);

  // tile kt in stage ST: substep 0 (reading substep 1 of this stage); wait
  // for tile kt+1's loads and every read of this stage; one barrier; tile
  // kt+2 starts loading into this stage; substep 1 (reading substep 0 of
  // tile kt+1 -- after the last tile, a harmless read of a settled stage)
  auto tile = [&](int kt, auto ST) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value;
    sub(TA{}, TA{}, stage(ST), I1{});
    wait_vm<0>();
    __syncthreads();
    if (kt + 2 < KT) gload(kt + 2, ST);
    sub(FA{}, TA{}, stage(std::integral_constant<int, st ^ 1>{}), I0{});
  };
  for (int kt = 0; kt < KT; kt += 2) {
    tile(kt, I0{});
    tile(kt + 1, I1{});
  }

  // the epilogue stages each wavefront's slab (32 x 68 floats) in the stage
  // buffers: wavefronts 0-3 in s0, 4-7 in s1
  __syncthreads();
  if constexpr (epi_f32<KIND>()) {
    static_assert(!BROWS, "bias along rows: bf16 outputs only");
    if (w < 4) epilogue_f32<KIND, true>(g, acc, reinterpret_cast<float *>(s0), w, lane, m0, n0, wm, wn);
    else epilogue_f32<KIND, true>(g, acc, reinterpret_cast<float *>(s1), w - 4, lane, m0, n0, wm, wn);
  } else {
    if (w < 4) epilogue<KIND, BROWS, true>(g, acc, reinterpret_cast<float *>(s0), w, lane, m0, n0, wm, wn);
    else epilogue<KIND, BROWS, true>(g, acc, reinterpret_cast<float *>(s1), w - 4, lane, m0, n0, wm, wn);
  }
}

// per-element epilogue (float32 path)
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
    k_gemm_bf16<KIND, BROWS><<<blocks, GW * 64, 0, s>>>(g);
  }
}

// Small GEMMs (the text / image K and V^T projections, the image MLP: M or N
// of a few hundred, a few dozen 256x256 tiles -- too few workgroups for the
// kernel above): 64x64 output tiles, four wavefronts of 32x32, operands
// straight from global memory / L2 into registers -- one 16-byte load per lane
// and operand per 16-deep K step, SPF steps ahead -- and one
// v_mfma_f32_32x32x16_bf16 per step.  As above the tile is computed transposed,
// so a lane stores runs of 4 consecutive columns of one output row.
constexpr int SBM = 64, SBN = 64, SPF = 4;
static_assert(64 % (16 * SPF) == 0, "K % 64 == 0 must make K / 16 a multiple of SPF");
template <int KIND, bool BROWS>
__global__ __launch_bounds__(256) void k_gemm_small(GemmDesc g) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int ncover = g.npad > g.N ? g.npad : g.N;
  const int tiles_n = (ncover + SBN - 1) / SBN;
  const int m0 = (int)(blockIdx.x / tiles_n) * SBM + (w >> 1) * 32;
  const int n0 = (int)(blockIdx.x % tiles_n) * SBN + (w & 1) * 32;
  // this lane's A row (output row) and B row (output column), clamped into the matrices
  const bf16 *pa = reinterpret_cast<const bf16 *>(g.A) + (long)min(m0 + l32, g.M - 1) * g.lda + half * 8;
  const bf16 *pb = reinterpret_cast<const bf16 *>(g.B) + (long)min(n0 + l32, g.N - 1) * g.ldb + half * 8;
  const int KS = g.K / 16;   // a multiple of SPF (K % 64 == 0)
  bf16x8 fa[SPF], fb[SPF];
#pragma unroll
  for (int i = 0; i < SPF; ++i) {
    const uint4 ua = ld16(pa + i * 16), ub = ld16(pb + i * 16);
    fa[i] = *reinterpret_cast<const bf16x8 *>(&ua);
    fb[i] = *reinterpret_cast<const bf16x8 *>(&ub);
  }
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int k0 = 0; k0 < KS; k0 += SPF) {
#pragma unroll
    for (int i = 0; i < SPF; ++i) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[i], acc, 0, 0, 0);
      if (k0 + i + SPF < KS) {
        const uint4 ua = ld16(pa + (k0 + i + SPF) * 16), ub = ld16(pb + (k0 + i + SPF) * 16);
        fa[i] = *reinterpret_cast<const bf16x8 *>(&ua);
        fb[i] = *reinterpret_cast<const bf16x8 *>(&ub);
      }
    }
  }
  // lane holds output row m0 + l32, columns n0 + 8 rb + 4 half + 0..3 (rb = 0..3)
  const int m = m0 + l32;
  if (m >= g.M) return;
  const bf16 *bias = reinterpret_cast<const bf16 *>(g.bias);
  const float rbias = BROWS && bias ? (float)bias[m] : 0.f;
  bf16 *crow = reinterpret_cast<bf16 *>(g.C) + (long)m * g.ldc;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int n = n0 + rb * 8 + half * 4;
    if (n >= ncover) continue;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nq = n + q < g.N ? n + q : g.N - 1;
      v[q] = acc[rb * 4 + q] + (BROWS ? rbias : (bias ? (float)bias[nq] : 0.f));
      if (KIND == OUT_GELU) v[q] = gelu_tanh(v[q]);
      if (KIND == OUT_BF16 && n + q < g.scale_cols) v[q] *= g.col_scale;
    }
    if (n + 4 <= g.N) {
      bf16x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = f2bf(v[q]);
      *reinterpret_cast<bf16x4 *>(crow + n) = o;
    } else {
      for (int q = 0; q < 4 && n + q < ncover; ++q) crow[n + q] = n + q < g.N ? f2bf(v[q]) : f2bf(0.f);
    }
  }
}

namespace {

hipError_t launch_gemm_one(const GemmDesc &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  // few tiles of the main kernel and a weight of at most 1536 x 1536 (larger
  // ones, re-read from L2 by every 64-row tile, run faster on the main kernel):
  // the small-GEMM kernel (bf16 / GELU outputs)
  if (!g.fp8 && !g.f32 && (g.kind == OUT_BF16 || g.kind == OUT_GELU) && !(g.bias_rows && g.kind != OUT_BF16) &&
      g.K % 64 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.ldc % 4 == 0 &&
      (long)((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN) < 64 &&
      (long)(g.M > g.N ? g.M : g.N) * g.K <= 1536L * 1536) {
    const int ncover = g.npad > g.N ? g.npad : g.N;
    const int blocks = ((g.M + SBM - 1) / SBM) * ((ncover + SBN - 1) / SBN);
    if (g.bias_rows) k_gemm_small<OUT_BF16, true><<<blocks, 256, 0, s>>>(g);
    else if (g.kind == OUT_GELU) k_gemm_small<OUT_GELU, false><<<blocks, 256, 0, s>>>(g);
    else k_gemm_small<OUT_BF16, false><<<blocks, 256, 0, s>>>(g);
    return hipGetLastError();
  }
  if (g.fp8) {
    if (g.K % 64 || !g.a_scale || !g.b_scale || g.f32) return hipErrorInvalidValue;
    if (g.b_per_col && !g.bias_rows) return hipErrorInvalidValue;   // per-column scales: token columns only
    if ((long)g.M * g.lda >= (1L << 31) || (long)g.N * g.ldb >= (1L << 31)) return hipErrorInvalidValue;
    const int blocks = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
    if (g.K % 256 == 0) {   // an even count of 128-deep K tiles
      if (g.bias_rows) {
        if (g.kind != OUT_BF16) return hipErrorInvalidValue;
        k_gemm_fp8w<OUT_BF16, true><<<blocks, GW * 64, 0, s>>>(g);
        return hipGetLastError();
      }
      switch (g.kind) {
        case OUT_BF16: k_gemm_fp8w<OUT_BF16, false><<<blocks, GW * 64, 0, s>>>(g); break;
        case OUT_F32: k_gemm_fp8w<OUT_F32, false><<<blocks, GW * 64, 0, s>>>(g); break;
        case OUT_GELU: k_gemm_fp8w<OUT_GELU, false><<<blocks, GW * 64, 0, s>>>(g); break;
        case OUT_RESID: k_gemm_fp8w<OUT_RESID, false><<<blocks, GW * 64, 0, s>>>(g); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    if (g.bias_rows) {
      if (g.kind != OUT_BF16) return hipErrorInvalidValue;
      k_gemm_fp8<OUT_BF16, true><<<blocks, GW * 64, 0, s>>>(g);
      return hipGetLastError();
    }
    switch (g.kind) {
      case OUT_BF16: k_gemm_fp8<OUT_BF16, false><<<blocks, GW * 64, 0, s>>>(g); break;
      case OUT_F32: k_gemm_fp8<OUT_F32, false><<<blocks, GW * 64, 0, s>>>(g); break;
      case OUT_GELU: k_gemm_fp8<OUT_GELU, false><<<blocks, GW * 64, 0, s>>>(g); break;
      case OUT_RESID: k_gemm_fp8<OUT_RESID, false><<<blocks, GW * 64, 0, s>>>(g); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (!g.f32 && (g.K % GBK)) return hipErrorInvalidValue;
  if (g.bias_rows && g.kind != OUT_BF16) return hipErrorInvalidValue;   // bias along rows: bf16 outputs
  // the bf16 kernel addresses A and B with 32-bit byte offsets
  if (!g.f32 && ((long)g.M * g.lda * 2 >= (1L << 31) || (long)g.N * g.ldb * 2 >= (1L << 31)))
    return hipErrorInvalidValue;
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

}  // namespace

// The bf16 and FP8 kernels address A and B with 32-bit byte offsets.  An
// operand of 2 GiB or more (the token side of a large batch: the FFN hidden
// state of several samples) is split here into launches over row or column
// slices, each operand slice below 2 GiB, each launch writing its own slice of
// the output.  The gated residual's gate is per batch sample, so row slices of
// that GEMM start at sample boundaries.
hipError_t launch_gemm(const GemmDesc &g, hipStream_t s) {
  if (g.f32 || g.M <= 0 || g.N <= 0) return launch_gemm_one(g, s);
  const long eb = g.fp8 ? 1 : 2;                       // operand element bytes
  const long ob = g.kind == OUT_F32 ? 4 : 2;           // C element bytes (not OUT_RESID)
  const long lim = (1L << 31) - 1;
  if (g.lda <= 0 || g.ldb <= 0) return hipErrorInvalidValue;
  if ((long)g.M * g.lda * eb > lim) {
    long rows = lim / (g.lda * eb);
    if (g.kind == OUT_RESID && g.gate)
      rows = g.rows_per_batch > 0 ? rows / g.rows_per_batch * g.rows_per_batch : 0;
    else
      rows = rows / GBM * GBM;
    if (rows <= 0) return hipErrorInvalidValue;
    for (long m0 = 0; m0 < g.M; m0 += rows) {
      GemmDesc c = g;
      c.M = (int)(g.M - m0 < rows ? g.M - m0 : rows);
      c.A = static_cast<const char *>(g.A) + m0 * g.lda * eb;
      if (g.kind == OUT_RESID) {
        c.X = g.X + m0 * g.ldx;
        if (g.gate) c.gate = g.gate + (m0 / g.rows_per_batch) * g.gate_bstride;
      } else {
        c.C = static_cast<char *>(g.C) + m0 * g.ldc * ob;
      }
      if (g.bias_rows && g.bias) c.bias = static_cast<const bf16 *>(g.bias) + m0;
      if (g.fp8 && g.a_per_row) c.a_scale = g.a_scale + m0;
      const hipError_t e = launch_gemm(c, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if ((long)g.N * g.ldb * eb > lim) {
    const long cols = lim / (g.ldb * eb) / GBN * GBN;
    if (cols <= 0) return hipErrorInvalidValue;
    for (long n0 = 0; n0 < g.N; n0 += cols) {
      GemmDesc c = g;
      c.N = (int)(g.N - n0 < cols ? g.N - n0 : cols);
      const bool last = n0 + cols >= g.N;
      c.B = static_cast<const char *>(g.B) + n0 * g.ldb * eb;
      if (g.kind == OUT_RESID) {
        c.X = g.X + n0;
        if (g.gate) c.gate = g.gate + n0;
      } else {
        c.C = static_cast<char *>(g.C) + n0 * ob;
      }
      if (!g.bias_rows && g.bias) c.bias = static_cast<const bf16 *>(g.bias) + n0;
      if (g.fp8 && g.b_per_col) c.b_scale = g.b_scale + n0;
      c.npad = last && g.npad > g.N ? (int)(g.npad - n0) : 0;
      c.scale_cols = g.scale_cols > n0 ? (int)(g.scale_cols - n0) : 0;
      const hipError_t e = launch_gemm_one(c, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_gemm_one(g, s);
}

}  // namespace wan
