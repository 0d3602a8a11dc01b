// Attention O = softmax(Q K^T / sqrt(hd)) V per (batch, head), no mask and no
// positional term: the full spatio-temporal self-attention and the text /
// image cross-attention of a DiT block ("Wan: Open and Advanced Large-Scale
// Video Generative Models (Wan 2.1)", section Diffusion Transformer; section
// I2V 架构扩展 for the decoupled image attention).
//
// bf16 path (hd = 128), flash style with an online softmax:
//  * a 512-thread workgroup owns 256 queries of one (batch, head): eight
//    wavefronts of 32 queries, two per SIMD;
//  * each wavefront interleaves its own matrix and vector work: the
//    exponentials of a tile are split in two halves, one laid between the
//    next tile's score MFMAs and one between the previous tile's PV MFMAs,
//    with LDS fragments read three MFMAs ahead (left to the compiler's
//    scheduler, the score MFMAs ran back to back on one-ahead reads and the
//    exponentials after them: 2% slower in the block);
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of ONE query, so the row max / row sum are
//    per-lane reductions plus one exchange between lanes l and l^32;
//  * O^T = V^T P^T: the probabilities are already in the B-operand layout.
//    The K rows of a tile sit in LDS in a permuted order (bits 2 and 3 of
//    the row index swapped within each 32-key block), which makes the 8
//    probabilities a lane feeds to one PV MFMA those of 8 consecutive keys;
//    V arrives transposed ([hd][key], written so by the projection GEMM), so
//    each V operand is one 16-byte ds_read_b128 of the natural V^T tile;
//  * K and V^T tiles of 64 keys go global -> LDS directly (buffer_load ...
//    lds), double-buffered, with XOR swizzles that keep every 16-lane group of
//    a 16-byte read on distinct banks; K runs one tile ahead of V;
//  * the score MFMAs start from an accumulator holding -m (m the running
//    max), so a score register already holds s - m.  The block's Q
//    projections write Q times log2(e)/sqrt(hd) (one rounding, in their
//    epilogue): a probability is then one v_exp_f32 of the register; for a
//    plain Q it is one multiply and one v_exp_f32;
//  * no row max in the steady state: the max is taken once, from the first
//    tile, and raised only when a tile's probabilities overflow 2^16 (seen in
//    the per-lane row sum); then that tile's max is taken, the accumulators
//    are rescaled and the tile's probabilities recomputed.  Probabilities
//    thus stay below 2^16, and the running sum below Lk * 2^16 (about 5e9 at
//    75600 keys: far inside float32's range).
#include <type_traits>

#include "attn.hpp"
#include "common.hpp"

namespace wan {

constexpr int AQ = 256;   // queries per workgroup: 8 wavefronts of 32
constexpr int AK = 64;    // keys per tile
constexpr int HD = 128;   // head dim
constexpr int KBW = 2;    // 1-KB blocks of a K (or V^T) tile each of the 8 wavefronts loads
constexpr int NA = 3;     // LDS fragment reads in flight ahead of their MFMA
constexpr float PMAX = 65536.0f;   // 2^16: probabilities above it raise the running max

WAN_DEV float other_half(float v) { return __shfl_xor(v, 32); }

typedef __attribute__((address_space(3))) void *lds_ptr;

// Row i of a K tile in LDS holds key ksig(i): bits 2 and 3 of i swapped.  A
// lane of half g then finds, in S^T registers r = 8 hf .. 8 hf + 7 of 32-key
// block kb, the keys kb*32 + 16 hf + 8 g + 0..7.
WAN_DEV int ksig(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
WAN_DEV int vswz(int row) { return (row >> 1) & 7; }   // 16-byte chunk XOR for 128-byte rows

// QS: q arrives multiplied by scale * log2(e) (a score is then already in
// log2 units); otherwise every score is multiplied by it before the exp2.
template <bool QS>
__global__ __launch_bounds__(512, 1) void k_attn_bf16(AttnDesc a) {
  // One LDS variable per stage: the compiler gives each its own alias scope,
  // so LDS reads of one stage need not wait for loads still landing in the
  // other (it cannot tell two halves of one array apart).  The steady-state
  // loop picks stages with compile-time parities.
  __shared__ __attribute__((aligned(16))) bf16 sK0[AK * HD];   // [row][hd], chunk ^ (row & 15)
  __shared__ __attribute__((aligned(16))) bf16 sK1[AK * HD];
  __shared__ __attribute__((aligned(16))) bf16 sV0[HD * AK];   // [hd][key], chunk ^ vswz(hd)
  __shared__ __attribute__((aligned(16))) bf16 sV1[HD * AK];
  // a stage is a std::integral_constant (steady state) or an int (the tail)
  auto kbuf = [&](auto P) -> bf16 * {
    if constexpr (std::is_integral_v<decltype(P)>) return P ? sK1 : sK0;
    else if constexpr (decltype(P)::value == 0) return sK0;
    else return sK1;
  };
  auto vbuf = [&](auto P) -> bf16 * {
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
  const int nqt = (a.Lq + AQ - 1) / AQ;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = bid % nqt, bh = bid / nqt;
  const int h = bh % a.H, b = bh / a.H;
  const int Lq = a.Lq, Lk = a.Lk;

  const bf16 *Qg = reinterpret_cast<const bf16 *>(a.q);
  const bf16 *Kg = reinterpret_cast<const bf16 *>(a.k);
  const bf16 *Vg = reinterpret_cast<const bf16 *>(a.vt);

  // ---- Q fragments (B operand of S^T = K Q^T): the lane holds
  // Q[q][st*16 + g*8 .. +8] of its query q = qrow
  // log2 units per score unit: 1 for a pre-scaled q, else scale * log2(e)
  const float c = QS ? 1.0f : a.scale * 1.4426950408889634f;
  const int qrow = qt * AQ + w * 32 + l32;
  bf16x8 qf[8];
  {
    const bool ok = qrow < Lq;
    const bf16 *qp = Qg + (long)(b * Lq + (ok ? qrow : 0)) * a.ldq + h * HD + g * 8;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint4 v = ok ? ld16(qp + st * 16) : make_uint4(0, 0, 0, 0);
      qf[st] = *reinterpret_cast<bf16x8 *>(&v);
    }
  }

  f32x16 o[4];   // O^T: head-dim rows t*32 .. +31 x the wavefront's 32 queries
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  // nm: -m in all 16 entries (the score MFMAs' initial accumulator); m is the
  // running max in score units (log2 units when QS)
  f32x16 nm;
#pragma unroll
  for (int r = 0; r < 16; ++r) nm[r] = 0.f;
  float l = 0.f;

  // ---- tile loaders: K tile = 64 keys x 16 chunks; V^T tile = 128 rows x 8 chunks
  const long vbase = (long)b * a.vt_bstride;
  // K tile: global -> LDS directly (buffer_load_dwordx4 ... lds).  The tile is
  // 16 blocks of 1 KB (4 rows each); wavefront w fills blocks w*KBW ..; lane i
  // lands at row blk*4 + i/16, physical chunk i%16; it fetches key ksig(row),
  // logical chunk (i%16) ^ (row & 15).  The descriptor spans exactly this
  // batch's Lk key rows, so rows past Lk read as zero.
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Kg + (long)b * Lk * a.ldk), 0, (int)((unsigned)Lk * (unsigned)a.ldk * 2u), 0x00020000);
  int kvoff[KBW];
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    const int row = (w * KBW + i) * 4 + (lane >> 4);    // LDS row of this lane's chunk
    const int chunk = (lane & 15) ^ (row & 15);
    kvoff[i] = (ksig(row) * (int)a.ldk + h * HD + chunk * 8) * 2;
  }
  auto gloadK = [&](int j, auto P) {
    const int rowb = j * AK * (int)a.ldk * 2;
    bf16 *dst = kbuf(P);
#pragma unroll
    for (int i = 0; i < KBW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr)(dst + (w * KBW + i) * 512), 16,
                                               kvoff[i] + rowb, 0, 0, 0);
  };
  // V^T tile: global -> LDS directly.  128 rows (hd) x 64 keys = 16 blocks of
  // 1 KB (8 rows each); wavefront w fills blocks w*KBW ..; lane i lands at row
  // blk*8 + i/8, physical chunk i%8 and fetches the logical chunk
  // (i%8) ^ vswz(row), i.e. keys 8*chunk .. +7 of the tile.  Columns past Lk
  // are read from the caller's zero padding.
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      (void *)Vg, 0, (int)((unsigned)(a.H * HD) * (unsigned)a.ldv * 2u), 0x00020000);
  int vvoff[KBW];
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    const int row = (w * KBW + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ vswz(row);
    vvoff[i] = (int)(((h * HD + row) * (long)a.ldv + vbase + chunk * 8) * 2);
  }
  auto gloadV = [&](int j, auto P) {
    const int colb = j * AK * 2;
    bf16 *dst = vbuf(P);
#pragma unroll
    for (int i = 0; i < KBW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr)(dst + (w * KBW + i) * 512), 16,
                                               vvoff[i] + colb, 0, 0, 0);
  };

  // per-lane LDS read offsets (elements); tile / buffer offsets are added as constants
  int koff[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) koff[st] = l32 * HD + (((st * 2 + g) ^ (l32 & 15)) * 8);
  int voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) voff[j] = l32 * AK + (((2 * j + g) ^ vswz(l32)) * 8);
  // LDS fragments: MFMA i = 2 st + kb of a score section (the two 32-key
  // chains alternate), MFMA i = (2 kb + hf) * 4 + t of a PV section
  auto kfr = [&](const bf16 *sk, int i) {
    return *reinterpret_cast<const bf16x8 *>(sk + (i & 1) * 32 * HD + koff[i >> 1]);
  };
  auto vfr = [&](const bf16 *sv, int i) {
    return *reinterpret_cast<const bf16x8 *>(sv + (i & 3) * 32 * AK + voff[i >> 2]);
  };

  const int ntiles = (Lk + AK - 1) / AK;

  // S^T - m of a tile (the first tile; the steady state interleaves these MFMAs)
  auto qk = [&](const bf16 *sk, f32x16 (&s)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr(sk, i), qf[i >> 1], i >> 1 ? s[i & 1] : nm,
                                                         0, 0, 0);
  };
  // keys past Lk -> -inf (last tile only)
  auto mask_tail = [&](f32x16 (&s)[2], int j) {
    if ((j + 1) * AK > Lk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * AK + kb * 32 + 16 * (r >> 3) + 8 * g + 4 * ((r >> 2) & 1) + (r & 3);
          if (key >= Lk) s[kb][r] = -INFINITY;
        }
    }
  };
  // row max of a score tile, merged across the two lane halves
  auto rowmax = [&](const f32x16 (&s)[2]) {
    float v = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, s[kb][r]);
    return fmaxf(v, other_half(v));
  };
  // One unit of a tile's probabilities: registers 2u, 2u+1 (u = 0..7) of a
  // 32-key block's centred scores sk -> exp2 -> bf16 pair u % 4 of pbk[u / 4]
  // (the B-operand layout of the PV MFMA), added to row-sum chain u % 2.  A
  // row sum adds the bf16-rounded probabilities, two per v_dot2 with (1, 1):
  // the normaliser then matches exactly the weights the PV MFMA uses.
  bf16x2 one2;
  one2[0] = (bf16)1.0f; one2[1] = (bf16)1.0f;
  auto punit = [&](const f32x16 &sk, int u, bf16x8 (&pbk)[2], float (&lsc)[2]) {
    const int hf = u >> 2, pp = u & 3;
    const float e0 = __builtin_amdgcn_exp2f(QS ? sk[2 * u] : sk[2 * u] * c);
    const float e1 = __builtin_amdgcn_exp2f(QS ? sk[2 * u + 1] : sk[2 * u + 1] * c);
    pbk[hf][2 * pp] = f2bf(e0);
    pbk[hf][2 * pp + 1] = f2bf(e1);
    bf16x2 pr;
    pr[0] = pbk[hf][2 * pp]; pr[1] = pbk[hf][2 * pp + 1];
    lsc[pp & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lsc[pp & 1], false);
  };
  // all probabilities of a tile and their row sum (the same units in the same order)
  auto probs = [&](const f32x16 (&s)[2], bf16x8 (&pb)[2][2], float &ls) {
    float lsc[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 8; ++u) punit(s[kb], u, pb[kb], lsc);
    ls = lsc[0] + lsc[1];
  };
  // lower every centred score of s by dm
  auto shift = [&](f32x16 (&s)[2], float dm) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] -= dm;
  };
  // a probability of this tile passed PMAX (or is not finite): raise the
  // running max to the tile's max, rescale the accumulators, recompute the
  // tile's probabilities; snxt (already scored against the old max) follows
  auto overflow = [&](f32x16 (&scur)[2], f32x16 (&snxt)[2], bool has_next, bf16x8 (&pb)[2][2],
                      float &ls) {
    if (__builtin_amdgcn_ballot_w64(!(ls <= PMAX)) == 0) return;
    const float dm = fmaxf(rowmax(scur), 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-dm * c);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) nm[r] -= dm;
    shift(scur, dm);
    if (has_next) shift(snxt, dm);
    probs(scur, pb, ls);
  };
  // O^T += V^T P^T (the last tile; the steady state interleaves these MFMAs)
  auto pv = [&](const bf16 *sv, const bf16x8 (&pb)[2][2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr(sv, i), pb[i >> 3][(i >> 2) & 1], o[i & 3],
                                                         0, 0, 0);
  };

  // Pipeline: K runs one tile ahead of V.  At the top of iteration j the LDS
  // holds K(j+1) in stage (j+1)&1 and V(j) in stage j&1; the centred scores
  // S(j) are in registers, and so are the probabilities of S(j)'s first
  // 32-key block.  Iteration j: K(j+2) and V(j+1) start loading into the
  // stages freed in iteration j-1; section 1: the 16 S(j+1) MFMAs, every
  // second one followed by one unit of S(j)'s second block; (rare) overflow:
  // raise the max; section 2: the 16 PV(j) MFMAs, every second one followed
  // by one unit of S(j+1)'s first block; wait for the loads; one barrier.
  // Each MFMA's fragment is read NA MFMAs ahead, and a scheduling barrier
  // after every MFMA keeps this order, so each wavefront keeps the matrix and
  // the vector unit busy together.
  constexpr std::integral_constant<int, 0> P0{};
  constexpr std::integral_constant<int, 1> P1{};
  gloadK(0, P0);
  if (ntiles > 1) gloadK(1, P1);
  gloadV(0, P0);
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): K(0), K(1), V(0) landed
  __syncthreads();
  f32x16 sa[2], sb[2];   // centred scores of the current / next tile
  bf16x8 pa[2], pn[2];   // probabilities of the first block of the current / next tile
  float la[2], ln[2];    // their row-sum chains
  {   // the first tile sets the running max exactly
    qk(sK0, sa);
    mask_tail(sa, 0);
    const float mx = rowmax(sa);
    shift(sa, mx);
#pragma unroll
    for (int r = 0; r < 16; ++r) nm[r] = -mx;
    la[0] = la[1] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) punit(sa[0], u, pa, la);
  }
  __syncthreads();   // every wavefront has read K(0): its buffer may be refilled

  // one pipelined iteration; tile j+1 exists; P is the parity of j; pc / lc:
  // probabilities and row-sum chains of S(j)'s first block, pnx / lnx the
  // same for S(j+1) (written here).  (load_k2: tile j+2 exists; mask_next:
  // tile j+1 is the last, possibly ragged, tile; both are constants in the
  // steady-state loop, so no branch stays there.)
  auto step = [&](auto P, int j, f32x16 (&scur)[2], f32x16 (&snxt)[2], bf16x8 (&pc)[2], float (&lc)[2],
                  bf16x8 (&pnx)[2], float (&lnx)[2], bool load_k2, bool mask_next) {
    const auto Q = other(P);
    const bf16 *sk = kbuf(Q);
    const bf16 *sv = vbuf(P);
    bf16x8 fr[NA + 1];
    // the first fragments are read before the tile loads are issued (their
    // LDS latency then overlaps the load issue)
#pragma unroll
    for (int i = 0; i < NA; ++i) fr[i] = kfr(sk, i);
    __builtin_amdgcn_sched_barrier(0);
    // both tile loads start at the top, so each has the whole iteration to
    // land before the wait at its end
    if (load_k2) gloadK(j + 2, P);   // buffer of K(j), read in iteration j-1
    gloadV(j + 1, Q);                // buffer of V(j-1), read in iteration j-1
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pt[2][2];                 // this tile's probabilities, the PV B operands
    pt[0][0] = pc[0]; pt[0][1] = pc[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {   // section 1
      if (i + NA < 16) fr[(i + NA) % (NA + 1)] = kfr(sk, i + NA);
      const int st = i >> 1, kb = i & 1;
      snxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (NA + 1)], qf[st], st ? snxt[kb] : nm,
                                                         0, 0, 0);
      if (i & 1) punit(scur[1], i >> 1, pt[1], lc);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (mask_next) mask_tail(snxt, j + 1);
    float ls = lc[0] + lc[1];
    overflow(scur, snxt, true, pt, ls);
    l += ls;
#pragma unroll
    for (int i = 0; i < NA; ++i) fr[i] = vfr(sv, i);
    lnx[0] = lnx[1] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {   // section 2
      if (i + NA < 16) fr[(i + NA) % (NA + 1)] = vfr(sv, i + NA);
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (NA + 1)], pt[i >> 3][(i >> 2) & 1],
                                                         o[i & 3], 0, 0, 0);
      if (i & 1) punit(snxt[0], i >> 1, pnx, lnx);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): K(j+2), V(j+1) landed, LDS reads done
    __syncthreads();
  };
  // the last tile: no next scores
  auto last = [&](auto P, f32x16 (&scur)[2], bf16x8 (&pc)[2], float (&lc)[2]) {
    bf16x8 pt[2][2];
    pt[0][0] = pc[0]; pt[0][1] = pc[1];
#pragma unroll
    for (int u = 0; u < 8; ++u) punit(scur[1], u, pt[1], lc);
    float ls = lc[0] + lc[1];
    overflow(scur, scur, false, pt, ls);
    l += ls;
    pv(vbuf(P), pt);
  };
  int j = 0;
  for (; j + 3 < ntiles; j += 2) {     // unrolled by two (score buffers and stages alternate);
    step(P0, j, sa, sb, pa, la, pn, ln, true, false);       // never computes the last tile's scores
    step(P1, j + 1, sb, sa, pn, ln, pa, la, true, false);
  }
  // the last 1 .. 3 tiles, one at a time with run-time stages; the current
  // scores are in sa
  for (; j + 1 < ntiles; ++j) {
    step(j & 1, j, sa, sb, pa, la, pn, ln, j + 2 < ntiles, j + 2 == ntiles);
    sa[0] = sb[0]; sa[1] = sb[1];
    pa[0] = pn[0]; pa[1] = pn[1];
    la[0] = ln[0]; la[1] = ln[1];
  }
  last(j & 1, sa, pa, la);

  // ---- normalise and store: lane holds O^T[hd = t*32 + (r/4)*8 + g*4 + r%4][q = qrow]
  const float inv = 1.0f / (l + other_half(l));
  if (qrow >= Lq) return;
  const long orow = (long)(b * Lq + qrow);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int hd0 = t * 32 + rb * 8 + g * 4;
      float v0 = o[t][rb * 4 + 0] * inv, v1 = o[t][rb * 4 + 1] * inv;
      float v2 = o[t][rb * 4 + 2] * inv, v3 = o[t][rb * 4 + 3] * inv;
      if (a.out_mode == 1) {
        *reinterpret_cast<float4 *>(a.acc32 + orow * (a.H * HD) + h * HD + hd0) = make_float4(v0, v1, v2, v3);
        continue;
      }
      if (a.out_mode == 2) {
        float4 p = *reinterpret_cast<const float4 *>(a.acc32 + orow * (a.H * HD) + h * HD + hd0);
        v0 += p.x; v1 += p.y; v2 += p.z; v3 += p.w;
      }
      bf16x4 ov;
      ov[0] = f2bf(v0); ov[1] = f2bf(v1); ov[2] = f2bf(v2); ov[3] = f2bf(v3);
      *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(a.o) + orow * a.ldo + h * HD + hd0) = ov;
    }
}

// float32 path: one wavefront per (batch, head, query); lanes stride over the
// keys with a per-lane online softmax, merged across the wavefront at the end.
// V is read untransposed: rows [B*Lk, ldv], head h at column h*hd.
template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(AttnDesc a) {
  const int lane = threadIdx.x & 63;
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long total = (long)a.B * a.H * a.Lq;
  if (wid >= total) return;
  const int qi = wid % a.Lq;
  const int bh = wid / a.Lq;
  const int h = bh % a.H, b = bh / a.H;
  const float *Q = reinterpret_cast<const float *>(a.q) + (long)(b * a.Lq + qi) * a.ldq + h * D;
  const float *K = reinterpret_cast<const float *>(a.k);
  const float *V = reinterpret_cast<const float *>(a.vt);
  float qv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { qv[d] = Q[d]; acc[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int j = lane; j < a.Lk; j += 64) {
    const float *kp = K + (long)(b * a.Lk + j) * a.ldk + h * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kp[d], s);
    s *= a.scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
    const float *vp = V + (long)(b * a.Lk + j) * a.ldv + h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vp[d], acc[d] * al);
    m = mn;
  }
  const float M = wave_max(m);
  const float f = (m == -INFINITY) ? 0.f : expf(m - M);
  const float lt = wave_sum(l * f);
  float *O = reinterpret_cast<float *>(a.o) + (long)(b * a.Lq + qi) * a.ldo + h * D;
  float *A32 = a.acc32 + (long)(b * a.Lq + qi) * (a.H * D) + h * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float v = wave_sum(acc[d] * f) / lt;
    if (lane == (d & 63)) {
      if (a.out_mode == 1) A32[d] = v;
      else if (a.out_mode == 2) O[d] = v + A32[d];
      else O[d] = v;
    }
  }
}

hipError_t launch_attention(const AttnDesc &a, hipStream_t s) {
  if (a.B <= 0 || a.H <= 0 || a.Lq <= 0 || a.Lk <= 0) return hipSuccess;
  if (a.f32) {
    const long waves = (long)a.B * a.H * a.Lq;
    const int blocks = (int)((waves + 3) / 4);
    if (a.hd == 64) k_attn_f32<64><<<blocks, 256, 0, s>>>(a);
    else if (a.hd == 128) k_attn_f32<128><<<blocks, 256, 0, s>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.hd != HD) return hipErrorInvalidValue;
  // K rows are addressed through a buffer descriptor with 32-bit byte offsets
  if ((long)a.Lk * a.ldk * 2 >= (1L << 31)) return hipErrorInvalidValue;
  if ((long)a.H * a.hd * a.ldv * 2 >= (1L << 31)) return hipErrorInvalidValue;
  if (a.vt_bstride < (a.Lk + AK - 1) / AK * AK) return hipErrorInvalidValue;
  const int nqt = (a.Lq + AQ - 1) / AQ;
  if (a.q_scaled) k_attn_bf16<true><<<a.B * a.H * nqt, 512, 0, s>>>(a);
  else k_attn_bf16<false><<<a.B * a.H * nqt, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace wan
