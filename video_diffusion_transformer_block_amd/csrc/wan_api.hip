// libwandit host side: argument validation, workspace carving and the launch
// sequence of the block and the step.  Every entry point validates all of its
// arguments before it enqueues anything.  See include/wan_dit.h for the ABI.
//
// Block sequence ("Wan: Open and Advanced Large-Scale Video Generative Models
// (Wan 2.1)", section Diffusion Transformer; "超越Sora！…Wan2.1", section 核心创新二):
//   modb = mod + bias_i
//   h  = LN(x)(1+scale1)+shift1                       [k_ln_mod]
//   q|k = h Wqk^T + b ;  V^T = Wv h^T + b               [GEMM, GEMM with swapped operands]
//   o  = softmax(q k^T/sqrt(hd)) v                      [flash attention]
//   x += gate1 * (o Wo^T + bo)                          [GEMM, residual epilogue]
//   hc = LN(x) ; qc = hc Wq^T + b ; kc, V^T_c from ctx   [k_ln_mod, GEMMs]
//   o  = Attn(qc, kc, vc) (+ Attn(qc, ki, vi) for I2V)   [attention]
//   x += o Wo_c^T + bo_c                                 [GEMM, residual epilogue]
//   h  = LN(x)(1+scale2)+shift2 ; u = GELU(h W1^T + b1)  [k_ln_mod, GEMM+GELU]
//   x += gate2 * (u W2^T + b2)                           [GEMM, residual epilogue]
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/wan_dit.h"
#include "attn8.hpp"
#include "kernels.hpp"

using namespace wan;

// Device scratch of the allocation-free block entry point
// (wan_dit_block_fwd_noalloc): its temporaries live in this file-scope array
// instead of a caller's workspace.  Every GPU the library runs on holds its
// own copy until the process ends.  In host code the array's name is only a
// stand-in, not a device address: the address comes from hipGetSymbolAddress,
// taken once per device with that device current (scratch_base below), and
// only that address is ever handed to kernels.
static __device__ __align__(256) char scratch[WAN_NOALLOC_SCRATCH_BYTES];

namespace {

// events the calling host thread asked to have recorded around its next
// self-attention launches (wan_set_attention_events); per thread, so calls
// from other threads are unaffected
thread_local hipEvent_t att_ev_start = nullptr, att_ev_stop = nullptr;

constexpr size_t ALIGN = 256;
size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }
long rup(long v, long a) { return (v + a - 1) / a * a; }

// ---- 8-bit attention: Int8 / E4M3 copies of q, k, V^T and the attention on them

// byte offsets of the quantised copies in a workspace: q8, qs, k8, ks, v8t, vs, end
void attn8_offsets(int B, int H, int Lq, int Lk, size_t off[7]) {
  const size_t d = (size_t)H * 128, Lkp = (size_t)rup(Lk, 64), nkb = Lkp / 64;
  const size_t sz[6] = {(size_t)B * Lq * d, (size_t)B * Lq * H * 4, (size_t)B * Lk * d,
                        (size_t)B * H * nkb * 4, d * B * Lkp, (size_t)B * d * 4};
  size_t o = 0;
  for (int i = 0; i < 6; ++i) {
    off[i] = o;
    o += up(sz[i], ALIGN);
  }
  off[6] = o;
}

// sizes the 8-bit kernels address with 32-bit buffer offsets
bool attn8_fits(int B, int H, int Lq, int Lk) {
  const long d = (long)H * 128;
  return (long)Lk * d < (1L << 31) && d * B * rup(Lk, 64) < (1L << 31) && (long)B * Lq < (1L << 31) / d;
}

Attn8Desc attn8_desc(const void *q8, const float *qs, const void *k8, const float *ks, const void *v8t,
                     const float *vs, void *o, int ldo, int B, int H, int Lq, int Lk, bool q_scaled) {
  Attn8Desc a;
  a.q8 = static_cast<const int8_t *>(q8); a.ldq8 = (long)H * 128; a.qs = qs;
  a.k8 = static_cast<const int8_t *>(k8); a.ldk8 = (long)H * 128; a.ks = ks;
  a.v8t = static_cast<const uint8_t *>(v8t); a.v8_bstride = rup(Lk, 64); a.ldv8 = (long)B * a.v8_bstride;
  a.vs = vs;
  a.o = o; a.ldo = ldo;
  a.B = B; a.H = H; a.Lq = Lq; a.Lk = Lk;
  a.alpha = q_scaled ? 1.0f : 1.4426950408889634f / sqrtf(128.0f);
  return a;
}

Attn8Quant attn8_quant(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv, int vt_bstride,
                       int B, int H, int Lq, int Lk, void *q8, float *qs, void *k8, float *ks, void *v8t,
                       float *vs) {
  Attn8Quant z;
  z.q = q; z.ldq = ldq; z.k = k; z.ldk = ldk; z.vt = vt; z.ldv = ldv; z.vt_bstride = vt_bstride;
  z.B = B; z.H = H; z.Lq = Lq; z.Lk = Lk;
  z.q8 = q8; z.ldq8 = (long)H * 128; z.qs = qs;
  z.k8 = k8; z.ldk8 = (long)H * 128; z.ks = ks;
  z.v8t = v8t; z.v8_bstride = rup(Lk, 64); z.ldv8 = (long)B * z.v8_bstride; z.vs = vs;
  return z;
}

// argument checks shared by the 8-bit entry points taking bf16 q, k, V^T
int attn8_check_inputs(int ldq, int ldk, int ldv, int vt_bstride, int B, int H, int Lq, int Lk) {
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0) return WAN_ERR_SHAPE;
  if (ldq < (long)H * 128 || ldk < (long)H * 128 || ldq % 8 || ldk % 8) return WAN_ERR_SHAPE;
  if (ldv % 8 || vt_bstride % 8 || vt_bstride < rup(Lk, 64) || (long)ldv < (long)B * vt_bstride)
    return WAN_ERR_SHAPE;
  if (!attn8_fits(B, H, Lq, Lk)) return WAN_ERR_SHAPE;
  return WAN_OK;
}


struct Layout {
  size_t modb, hid, h, qk, vt, o, qc, kc, vtc, ki, vti, acc32, u;   // block
  size_t mod, x, P, pw, img1, img2, imgc;                           // step
  size_t aq, as;                                                    // FP8 activations
  size_t a8;                                                        // 8-bit attention copies
  size_t total;
  long Lp, Lcp, Lip;
  int Kp;
};

Layout make_layout(const wan_cfg_t &c, int B, long L, bool step, bool fp8 = false) {
  Layout y;
  memset(&y, 0, sizeof(y));
  const bool f32 = c.dtype == WAN_F32;
  const size_t es = f32 ? 4 : 2;
  const long d = c.dim, F = c.ffn, Lc = c.text_len, Li = c.img_len;
  y.Lp = rup(L, 64);
  y.Lcp = rup(Lc, 64);
  y.Lip = rup(Li > 0 ? Li : 1, 64);
  y.Kp = (int)rup(4L * c.in_ch, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes, ALIGN); return o; };
  y.modb = take(B * 6 * d * 4);
  y.hid = take(B * (d + c.freq_dim) * 4);
  y.h = take(B * L * d * es);
  y.qk = take(B * L * (f32 ? 3 : 2) * d * es);
  y.vt = take(f32 ? 0 : d * B * y.Lp * es);
  y.o = take(B * L * d * es);
  y.qc = take(B * L * d * es);
  y.kc = take(B * Lc * (f32 ? 2 : 1) * d * es);
  y.vtc = take(f32 ? 0 : d * B * y.Lcp * es);
  y.ki = take(Li ? B * Li * (f32 ? 2 : 1) * d * es : 0);
  y.vti = take(Li && !f32 ? d * B * y.Lip * es : 0);
  y.acc32 = take(Li ? B * L * d * 4 : 0);
  y.u = take(B * L * F * es);
  if (step) {
    y.mod = take(B * 6 * d * 4);
    y.x = take(B * L * d * 4);
    y.P = take(B * L * y.Kp * es);
    y.pw = take(d * y.Kp * es);
    y.img1 = take(Li ? B * Li * d * es : 0);
    y.img2 = take(Li ? B * Li * d * es : 0);
    y.imgc = take(Li ? B * Li * d * es : 0);
  }
  if (fp8) {   // E4M3 codes of one activation (the widest: FFN hidden) + per-token scales
    y.aq = take(B * L * (F > d ? F : d));
    y.as = take(B * L * 4);
  }
  if (c.attn8) {   // Int8 q, k and E4M3 V^T of the self-attention, with their scales
    size_t o8[7];
    attn8_offsets(B, c.heads, (int)L, (int)L, o8);
    y.a8 = take(o8[6]);
  }
  y.total = off;
  return y;
}

// Cross-attention K/V cache: one region per block holding the text keys and
// V^T (and, for I2V, the image pair) exactly as the block would project them.
struct KvLayout {
  size_t kc, vtc, ki, vti, per_block;
};

KvLayout kv_layout(const wan_cfg_t &c, int B) {
  KvLayout k;
  const bool f32 = c.dtype == WAN_F32;
  const size_t es = f32 ? 4 : 2;
  const long d = c.dim, Lc = c.text_len, Li = c.img_len;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes, ALIGN); return o; };
  k.kc = take(B * Lc * (f32 ? 2 : 1) * d * es);
  k.vtc = take(f32 ? 0 : d * B * rup(Lc, 64) * es);
  k.ki = take(Li ? B * Li * (f32 ? 2 : 1) * d * es : 0);
  k.vti = take(Li && !f32 ? d * B * rup(Li, 64) * es : 0);
  k.per_block = off;
  return k;
}

// where a block finds its cross-attention keys / values
struct KvPtrs {
  const void *kc, *vtc, *ki, *vti;
};

// Packed FP8 weights of one block: six float32 dequantisation scales (QKV,
// SA out, CA query, CA out, FFN up, FFN down), six running-maximum words
// used while quantising, then the six E4M3 weight tensors [out, in].
struct Fp8Layout {
  size_t sc, amax, w[6], total;
  long n[6];   // elements of each weight
};

Fp8Layout fp8_layout(const wan_cfg_t &c) {
  Fp8Layout q;
  const long d = c.dim, F = c.ffn;
  const long n[6] = {3 * d * d, d * d, d * d, d * d, F * d, d * F};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes, ALIGN); return o; };
  q.sc = take(6 * 4);
  q.amax = take(6 * 4);
  for (int i = 0; i < 6; ++i) {
    q.n[i] = n[i];
    q.w[i] = take((size_t)n[i]);
  }
  q.total = off;
  return q;
}

// FP8 operands of a block run: the packed weights and the activation buffers
struct Fp8Ptrs {
  const uint8_t *w[6];   // qkv, sa_wo, ca_wq, ca_wo, ffn_w1, ffn_w2
  const float *sc;       // [6]
  uint8_t *aq;           // activation codes
  float *as;             // per-token scales
};

int check_cfg(const wan_cfg_t *c) {
  if (!c) return WAN_ERR_NULL;
  if (c->dtype != WAN_F32 && c->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (c->dim <= 0 || c->heads <= 0 || c->head_dim <= 0 || c->ffn <= 0 || c->n_blocks < 0 ||
      c->in_ch <= 0 || c->out_ch <= 0 || c->freq_dim <= 0 || c->text_len <= 0 || c->img_len < 0)
    return WAN_ERR_SHAPE;
  if ((long)c->heads * c->head_dim != c->dim) return WAN_ERR_SHAPE;
  if (c->freq_dim % 2) return WAN_ERR_SHAPE;
  if (!(c->eps > 0.f) || !isfinite(c->eps)) return WAN_ERR_SHAPE;
  if (c->attn8 != 0 && c->attn8 != 1) return WAN_ERR_CONFIG;
  if (c->attn8 && c->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (c->dtype == WAN_BF16) {
    // MFMA tiles: K of every GEMM a multiple of 64; attention head dim 128
    if (c->head_dim != 128 || c->ffn % 64 || c->freq_dim % 8) return WAN_ERR_SHAPE;
    if (c->img_len > 0 && (c->img_feat <= 0 || c->img_feat % 64)) return WAN_ERR_SHAPE;
  } else {
    if (c->head_dim != 64 && c->head_dim != 128) return WAN_ERR_SHAPE;
    if (c->dim % 4 || c->freq_dim % 4) return WAN_ERR_SHAPE;
    if (c->img_len > 0 && (c->img_feat <= 0 || c->img_feat % 4)) return WAN_ERR_SHAPE;
  }
  return WAN_OK;
}

int check_dims(const wan_cfg_t &c, int B, int lat_f, int Hp, int Wp) {
  if (B <= 0 || B > 8 || lat_f <= 0 || Hp <= 0 || Wp <= 0) return WAN_ERR_SHAPE;
  const long L = (long)lat_f * Hp * Wp;
  if ((long)B * L > (1L << 30)) return WAN_ERR_SHAPE;
  if (c.attn8 && !attn8_fits(B, c.heads, (int)L, (int)L)) return WAN_ERR_SHAPE;
  if (c.dtype == WAN_BF16) {
    // the MFMA kernels address operands with 32-bit byte offsets: a GEMM
    // operand of 2 GiB or more is split at sample boundaries, so one sample's
    // (the FFN hidden state, Q||K) must fit; the self-attention's V^T of all
    // samples is one operand
    const long wmax = c.ffn > 2L * c.dim ? c.ffn : 2L * c.dim;
    if (L * wmax * 2 >= (1L << 31)) return WAN_ERR_SHAPE;
    if ((long)c.dim * B * rup(L, 64) * 2 >= (1L << 31)) return WAN_ERR_SHAPE;
  }
  return WAN_OK;
}

hipStream_t S(void *s) { return reinterpret_cast<hipStream_t>(s); }

#define WAN_TRY(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return WAN_ERR_HIP;  \
  } while (0)

const char *off(const void *p, long elems, size_t es) {
  return reinterpret_cast<const char *>(p) + elems * (long)es;
}

GemmDesc gemm(const void *A, long lda, const void *B, long ldb, int M, int N, int K,
              const void *bias, int kind, void *C, long ldc, int f32) {
  GemmDesc g;
  memset(&g, 0, sizeof(g));
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
  g.bias = bias; g.kind = kind; g.C = C; g.ldc = ldc; g.f32 = f32;
  return g;
}

GemmDesc resid(const void *A, long lda, const void *W, int M, int N, int K, const void *bias,
               float *X, const float *gate, long gate_bs, int rows_per_batch, int f32) {
  GemmDesc g = gemm(A, lda, W, K, M, N, K, bias, OUT_RESID, nullptr, 0, f32);
  g.X = X; g.ldx = N; g.gate = gate; g.gate_bstride = gate_bs; g.rows_per_batch = rows_per_batch;
  return g;
}

// y[B*Lk, d] = src W^T + b ; V^T[d, b*ldvb + j] = (src_b Wv^T + bv)^T for a K/V source.
int kv_project(const wan_cfg_t &c, int B, int Lk, const void *src, const void *wkv,
               const void *bkv, char *kbuf, char *vtbuf, long ldvb, hipStream_t s) {
  const int d = c.dim;
  const int f32 = c.dtype == WAN_F32;
  const size_t es = f32 ? 4 : 2;
  if (f32) {   // one GEMM, keys and values side by side: [B*Lk, 2d]
    WAN_TRY(launch_gemm(gemm(src, d, wkv, d, B * Lk, 2 * d, d, bkv, OUT_BF16, kbuf, 2 * d, 1), s));
    return WAN_OK;
  }
  WAN_TRY(launch_gemm(gemm(src, d, wkv, d, B * Lk, d, d, bkv, OUT_BF16, kbuf, d, 0), s));
  for (int b = 0; b < B; ++b) {
    GemmDesc g = gemm(off(wkv, (long)d * d, es), d, off(src, (long)b * Lk * d, es), d, d, Lk, d,
                      off(bkv, d, es), OUT_BF16, vtbuf + (long)b * ldvb * es, (long)B * ldvb, 0);
    g.bias_rows = 1;
    g.npad = (int)ldvb;   // keys Lk .. ldvb-1 of this batch segment are zero
    WAN_TRY(launch_gemm(g, s));
  }
  return WAN_OK;
}

// the output's first `cols` columns times log2(e)/sqrt(hd): a query the bf16
// attention kernel reads pre-scaled (AttnDesc::q_scaled)
GemmDesc qscaled(GemmDesc g, int cols, int hd) {
  g.scale_cols = cols;
  g.col_scale = 1.4426950408889634f / sqrtf((float)hd);
  return g;
}

// the same GEMM on E4M3 operands: acc * a_scale[m or 0] * b_scale[n or 0]
GemmDesc fp8(GemmDesc g, const float *as, int a_per_row, const float *bs, int b_per_col) {
  g.fp8 = 1;
  g.a_scale = as; g.a_per_row = a_per_row;
  g.b_scale = bs; g.b_per_col = b_per_col;
  return g;
}

AttnDesc attn(const void *q, long ldq, const void *k, long ldk, const void *v, long ldv,
              long vbs, void *o, long ldo, int B, int H, int Lq, int Lk, int hd, int f32,
              int q_scaled = 0) {
  AttnDesc a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.vt = v; a.ldv = ldv; a.vt_bstride = vbs;
  a.o = o; a.ldo = ldo; a.B = B; a.H = H; a.Lq = Lq; a.Lk = Lk; a.hd = hd;
  a.scale = 1.0f / sqrtf((float)hd); a.f32 = f32; a.q_scaled = q_scaled;
  return a;
}

// One block.  Cross-attention keys / values come from `cached` when it is
// given, else they are projected from ctx (and img) into the workspace.  With
// `q8` the six Linear layers run on E4M3 operands: each bf16 activation is
// quantised per token right before the GEMM that reads it ([Note] Infra /
// 推理优化: FP8 GEMM); the text / image K/V projections stay bf16.
int block_run(const wan_cfg_t &c, float *x, int B, long L, const float *mod,
              const wan_block_weights_t &w, const void *ctx, const void *img, const KvPtrs *cached,
              char *ws, const Layout &y, hipStream_t s, const Fp8Ptrs *q8 = nullptr) {
  const int d = c.dim, F = c.ffn, H = c.heads, hd = c.head_dim, Lc = c.text_len, Li = c.img_len;
  const int f32 = c.dtype == WAN_F32;
  const size_t es = f32 ? 4 : 2;
  const int M = (int)(B * L);
  float *modb = reinterpret_cast<float *>(ws + y.modb);
  char *h = ws + y.h, *qk = ws + y.qk, *vt = ws + y.vt, *o = ws + y.o, *qc = ws + y.qc;
  char *kc = ws + y.kc, *vtc = ws + y.vtc, *ki = ws + y.ki, *vti = ws + y.vti, *u = ws + y.u;
  float *acc32 = reinterpret_cast<float *>(ws + y.acc32);

  // LayerNorm (+ modulate) of x into h; with q8 into the E4M3 activation
  // buffer instead (fused when the width allows)
  auto ln = [&](int shift_off, int scale_off, int has_mod) -> hipError_t {
    if (q8 && ln_mod_fp8_supported(d))
      return launch_ln_mod_fp8(x, M, (int)L, d, modb, 6 * d, shift_off, scale_off, has_mod, c.eps,
                               q8->aq, q8->as, s);
    hipError_t e = launch_ln_mod(x, M, (int)L, d, modb, 6 * d, shift_off, scale_off, has_mod, c.eps,
                                 h, f32, s);
    if (e != hipSuccess || !q8) return e;
    return launch_quant_rows_fp8(h, M, d, d, q8->aq, d, q8->as, s);
  };
  // y = act W^T + b with the residual / GELU / plain epilogue g; on E4M3
  // operands with q8 (act quantised per token first unless `quantised`)
  auto linear = [&](GemmDesc g, int wi, bool quantised) -> hipError_t {
    if (!q8) return launch_gemm(g, s);
    if (!quantised) {
      hipError_t e = launch_quant_rows_fp8(g.A, M, g.K, g.lda, q8->aq, g.K, q8->as, s);
      if (e != hipSuccess) return e;
    }
    g.A = q8->aq; g.lda = g.K;
    g.B = q8->w[wi]; g.ldb = g.K;
    return launch_gemm(fp8(g, q8->as, 1, q8->sc + wi, 0), s);
  };

  // self-attention of the bf16 paths on q | k in qk and V^T in vt: bf16 with
  // the pre-scaled query, or (cfg attn8) quantised to Int8 / E4M3 and run by
  // the 8-bit kernel ([Note] Infra / 推理优化: 8-bit FlashAttention)
  auto self_attn = [&]() -> hipError_t {
    if (!c.attn8)
      return launch_attention(attn(qk, 2 * d, off(qk, d, es), 2 * d, vt, (long)B * y.Lp, y.Lp, o, d, B, H,
                                   (int)L, (int)L, hd, 0, 1), s);
    char *a8 = ws + y.a8;
    size_t o8[7];
    attn8_offsets(B, H, (int)L, (int)L, o8);
    float *qs8 = (float *)(a8 + o8[1]), *ks8 = (float *)(a8 + o8[3]), *vs8 = (float *)(a8 + o8[5]);
    hipError_t e = launch_quant_attn8(attn8_quant(qk, 2 * d, off(qk, d, es), 2 * d, vt, (int)((long)B * y.Lp),
                                                  (int)y.Lp, B, H, (int)L, (int)L, a8 + o8[0], qs8,
                                                  a8 + o8[2], ks8, a8 + o8[4], vs8), s);
    if (e != hipSuccess) return e;
    return launch_attention8(attn8_desc(a8 + o8[0], qs8, a8 + o8[2], ks8, a8 + o8[4], vs8, o, d, B, H,
                                        (int)L, (int)L, false), s);
  };

  // the self-attention, between the measurement events when the thread has set them
  auto self_attn_timed = [&]() -> hipError_t {
    if (att_ev_start) {
      const hipError_t e = hipEventRecord(att_ev_start, s);
      if (e != hipSuccess) return e;
    }
    const hipError_t e = self_attn();
    if (e != hipSuccess || !att_ev_stop) return e;
    return hipEventRecord(att_ev_stop, s);
  };

  WAN_TRY(launch_mod_combine(mod, w.mod_bias, modb, B, 6 * d, s));
  // ---- self-attention branch
  WAN_TRY(ln(0, d, 1));
  if (f32) {
    WAN_TRY(launch_gemm(gemm(h, d, w.sa_wqkv, d, M, 3 * d, d, w.sa_bqkv, OUT_BF16, qk, 3 * d, 1), s));
    WAN_TRY(launch_attention(attn(qk, 3 * d, off(qk, d, es), 3 * d, off(qk, 2 * d, es), 3 * d, 0,
                                  o, d, B, H, (int)L, (int)L, hd, 1), s));
  } else if (q8) {
    // with the 8-bit attention the query stays unscaled (it is quantised per token)
    GemmDesc gqk = gemm(q8->aq, d, q8->w[0], d, M, 2 * d, d, w.sa_bqkv, OUT_BF16, qk, 2 * d, 0);
    WAN_TRY(launch_gemm(fp8(c.attn8 ? gqk : qscaled(gqk, d, hd), q8->as, 1, q8->sc + 0, 0), s));
    for (int b = 0; b < B; ++b) {   // V^T = Wv h_b^T: weight scale per tensor, token scale per column
      GemmDesc g = gemm(q8->w[0] + 2L * d * d, d, q8->aq + (long)b * L * d, d, d, (int)L, d,
                        off(w.sa_bqkv, 2 * d, es), OUT_BF16, vt + b * y.Lp * es, (long)B * y.Lp, 0);
      g.bias_rows = 1;
      g.npad = (int)y.Lp;
      WAN_TRY(launch_gemm(fp8(g, q8->sc + 0, 0, q8->as + (long)b * L, 1), s));
    }
    WAN_TRY(self_attn_timed());
  } else {
    GemmDesc gqk = gemm(h, d, w.sa_wqkv, d, M, 2 * d, d, w.sa_bqkv, OUT_BF16, qk, 2 * d, 0);
    WAN_TRY(launch_gemm(c.attn8 ? gqk : qscaled(gqk, d, hd), s));
    for (int b = 0; b < B; ++b) {
      GemmDesc g = gemm(off(w.sa_wqkv, 2L * d * d, es), d, off(h, (long)b * L * d, es), d, d,
                        (int)L, d, off(w.sa_bqkv, 2 * d, es), OUT_BF16, vt + b * y.Lp * es,
                        (long)B * y.Lp, 0);
      g.bias_rows = 1;
      g.npad = (int)y.Lp;   // keys L .. Lp-1 of this batch segment are zero
      WAN_TRY(launch_gemm(g, s));
    }
    WAN_TRY(self_attn_timed());
  }
  WAN_TRY(linear(resid(o, d, w.sa_wo, M, d, d, w.sa_bo, x, modb + 2 * d, 6 * d, (int)L, f32), 1,
                 false));

  // ---- cross-attention branch (pre-LN without modulation, ungated)
  WAN_TRY(ln(0, 0, 0));
  GemmDesc gq = gemm(h, d, w.ca_wq, d, M, d, d, w.ca_bq, OUT_BF16, qc, d, f32);
  WAN_TRY(linear(f32 ? gq : qscaled(gq, d, hd), 2, true));
  int st;
  if (cached) {
    kc = (char *)cached->kc; vtc = (char *)cached->vtc; ki = (char *)cached->ki; vti = (char *)cached->vti;
  } else {
    st = kv_project(c, B, Lc, ctx, w.ca_wkv, w.ca_bkv, kc, vtc, y.Lcp, s);
    if (st) return st;
  }
  const long kld = f32 ? 2 * d : d;
  AttnDesc at = f32 ? attn(qc, d, kc, kld, off(kc, d, es), kld, 0, o, d, B, H, (int)L, Lc, hd, 1)
                    : attn(qc, d, kc, kld, vtc, (long)B * y.Lcp, y.Lcp, o, d, B, H, (int)L, Lc, hd, 0, 1);
  if (Li > 0) {
    if (!cached) {
      st = kv_project(c, B, Li, img, w.ca_wkv_img, w.ca_bkv_img, ki, vti, y.Lip, s);
      if (st) return st;
    }
    at.out_mode = 1;
    at.acc32 = acc32;
    WAN_TRY(launch_attention(at, s));
    AttnDesc ai = f32 ? attn(qc, d, ki, kld, off(ki, d, es), kld, 0, o, d, B, H, (int)L, Li, hd, 1)
                      : attn(qc, d, ki, kld, vti, (long)B * y.Lip, y.Lip, o, d, B, H, (int)L, Li, hd, 0, 1);
    ai.out_mode = 2;
    ai.acc32 = acc32;
    WAN_TRY(launch_attention(ai, s));
  } else {
    WAN_TRY(launch_attention(at, s));
  }
  WAN_TRY(linear(resid(o, d, w.ca_wo, M, d, d, w.ca_bo, x, nullptr, 0, (int)L, f32), 3, false));

  // ---- FFN branch
  WAN_TRY(ln(3 * d, 4 * d, 1));
  WAN_TRY(linear(gemm(h, d, w.ffn_w1, d, M, F, d, w.ffn_b1, OUT_GELU, u, F, f32), 4, true));
  WAN_TRY(linear(resid(u, F, w.ffn_w2, M, d, F, w.ffn_b2, x, modb + 5 * d, 6 * d, (int)L, f32), 5,
                 false));
  return WAN_OK;
}

// every pointer the block reads; with fp8 the six quantised weights are not read
int check_block_weights(const wan_cfg_t &c, const wan_block_weights_t *w, bool fp8 = false) {
  if (!w) return WAN_ERR_NULL;
  const void *req[] = {w->sa_bqkv, w->sa_bo, w->ca_bq, w->ca_wkv, w->ca_bkv, w->ca_bo, w->ffn_b1,
                       w->ffn_b2, w->mod_bias};
  for (const void *p : req)
    if (!p) return WAN_ERR_NULL;
  if (!fp8 && (!w->sa_wqkv || !w->sa_wo || !w->ca_wq || !w->ca_wo || !w->ffn_w1 || !w->ffn_w2))
    return WAN_ERR_NULL;
  if (c.img_len > 0 && (!w->ca_wkv_img || !w->ca_bkv_img)) return WAN_ERR_CONFIG;
  return WAN_OK;
}

// I2V image context: three Linear layers with GELU between them
// ([Note] I2V 架构扩展: CLIP features through a 3-layer MLP); returns its
// [B*Li, d] output in the workspace regions img1 / img2 / imgc.
int image_context(const wan_cfg_t &c, int B, const void *clip, const wan_model_weights_t &w,
                  char *img1, char *img2, char *imgc, hipStream_t s) {
  const int d = c.dim, f32 = c.dtype == WAN_F32;
  const int Mi = B * c.img_len;
  WAN_TRY(launch_gemm(gemm(clip, c.img_feat, w.img_w1, c.img_feat, Mi, d, c.img_feat, w.img_b1,
                           OUT_GELU, img1, d, f32), s));
  WAN_TRY(launch_gemm(gemm(img1, d, w.img_w2, d, Mi, d, d, w.img_b2, OUT_GELU, img2, d, f32), s));
  WAN_TRY(launch_gemm(gemm(img2, d, w.img_w3, d, Mi, d, d, w.img_b3, OUT_BF16, imgc, d, f32), s));
  return WAN_OK;
}

// every weight the step reads (image MLP only when `need_img`; with fp8 the
// blocks' six quantised weights are not read)
int check_model_weights(const wan_cfg_t &c, const wan_model_weights_t *w, bool need_img,
                        bool fp8 = false) {
  if (!w) return WAN_ERR_NULL;
  if (!w->patch_w || !w->patch_b || !w->head_w || !w->head_b || !w->tmlp.w1 || !w->tmlp.b1 ||
      !w->tmlp.w2 || !w->tmlp.b2)
    return WAN_ERR_NULL;
  if (c.n_blocks > 0 && !w->blocks) return WAN_ERR_NULL;
  int st;
  for (int i = 0; i < c.n_blocks; ++i)
    if ((st = check_block_weights(c, &w->blocks[i], fp8))) return st;
  if (need_img && (!w->img_w1 || !w->img_b1 || !w->img_w2 || !w->img_b2 || !w->img_w3 || !w->img_b3))
    return WAN_ERR_CONFIG;
  return WAN_OK;
}

// the FP8 operands of block i of a model's packed weights (n_blocks regions)
Fp8Ptrs fp8_block_ptrs(const wan_cfg_t &c, const char *qbuf, int i, char *ws, const Layout &y) {
  const Fp8Layout ql = fp8_layout(c);
  const char *qb = qbuf + (size_t)i * ql.total;
  Fp8Ptrs q8;
  for (int k = 0; k < 6; ++k) q8.w[k] = (const uint8_t *)(qb + ql.w[k]);
  q8.sc = (const float *)(qb + ql.sc);
  q8.aq = (uint8_t *)ws + y.aq;
  q8.as = (float *)(ws + y.as);
  return q8;
}

// patchify -> t-MLP -> (image context) -> blocks -> head + unpatchify.  With
// `cache` the blocks read their cross-attention K/V from it (ctx / clip unused);
// with `q8buf` (a model's packed FP8 weights) every block runs its Linear
// layers in FP8.
int step_run(const wan_cfg_t &c, const float *latent, const float *t, int B, int lat_f, int H8,
             int W8, const void *ctx, const void *clip, const char *cache,
             const wan_model_weights_t &w, float *out, char *wsb, const Layout &y, hipStream_t s,
             const char *q8buf = nullptr) {
  const int d = c.dim, f32 = c.dtype == WAN_F32;
  const int Hp = H8 / 2, Wp = W8 / 2;
  const long L = (long)lat_f * Hp * Wp;
  float *x = reinterpret_cast<float *>(wsb + y.x);
  float *mod = reinterpret_cast<float *>(wsb + y.mod);
  const int M = (int)(B * L);
  // patchify: gather the (1,2,2) patches, then one GEMM against the padded Conv3d weight
  WAN_TRY(launch_patch_gather(latent, B, c.in_ch, lat_f, H8, W8, y.Kp, wsb + y.P, f32, s));
  WAN_TRY(launch_pad_rows(w.patch_w, d, 4 * c.in_ch, y.Kp, wsb + y.pw, f32, s));
  WAN_TRY(launch_gemm(gemm(wsb + y.P, y.Kp, wsb + y.pw, y.Kp, M, d, y.Kp, w.patch_b, OUT_F32, x, d,
                           f32), s));
  // shared timestep MLP
  WAN_TRY(launch_tmlp(t, B, c.freq_dim, d, w.tmlp.w1, w.tmlp.b1, w.tmlp.w2, w.tmlp.b2,
                      reinterpret_cast<float *>(wsb + y.hid), mod, f32, s));
  int st;
  const void *img = nullptr;
  if (c.img_len > 0 && !cache) {
    if ((st = image_context(c, B, clip, w, wsb + y.img1, wsb + y.img2, wsb + y.imgc, s))) return st;
    img = wsb + y.imgc;
  }
  const KvLayout kl = kv_layout(c, B);
  for (int i = 0; i < c.n_blocks; ++i) {
    KvPtrs kp;
    const KvPtrs *pk = nullptr;
    if (cache) {
      const char *base = cache + (size_t)i * kl.per_block;
      kp = {base + kl.kc, base + kl.vtc, base + kl.ki, base + kl.vti};
      pk = &kp;
    }
    Fp8Ptrs q8;
    if (q8buf) q8 = fp8_block_ptrs(c, q8buf, i, wsb, y);
    st = block_run(c, x, B, L, mod, w.blocks[i], ctx, img, pk, wsb, y, s, q8buf ? &q8 : nullptr);
    if (st) return st;
  }
  WAN_TRY(launch_head_unpatchify(x, B, lat_f, Hp, Wp, d, w.head_w, w.head_b, c.out_ch, out, f32, s));
  return WAN_OK;
}

// latent geometry of a step
int check_step_dims(const wan_cfg_t &c, int B, int lat_f, int H8, int W8) {
  if (H8 <= 0 || W8 <= 0 || H8 % 2 || W8 % 2) return WAN_ERR_SHAPE;
  return check_dims(c, B, lat_f, H8 / 2, W8 / 2);
}

size_t sample_extra(int B, int out_ch, long plane, size_t *t_off, size_t *v_off, size_t base) {
  *t_off = base;
  *v_off = *t_off + up((size_t)B * 4, ALIGN);
  return *v_off + up((size_t)B * out_ch * plane * 4, ALIGN);
}

// n_steps Euler steps of the cached step (see wan_sample_fwd); q8buf: FP8 blocks
int sample_run(const wan_cfg_t &c, float *latent, int B, int lat_f, int H8, int W8, int n_steps,
               int guided, float scale, const char *kv_cache, const wan_model_weights_t &w, char *wsb,
               const Layout &y, size_t t_off, size_t v_off, hipStream_t s, const char *q8buf = nullptr) {
  float *tb = reinterpret_cast<float *>(wsb + t_off);
  float *vel = reinterpret_cast<float *>(wsb + v_off);
  const long plane = (long)lat_f * H8 * W8;
  // flow time tau_k = k / n from noise (0) to data (1); the model's timestep
  // input is 1000 tau_k; one Euler step of length 1/n per evaluation
  const float dt = (float)(1.0 / n_steps);
  for (int k = 0; k < n_steps; ++k) {
    WAN_TRY(launch_fill(tb, B, (float)(1000.0 * k / n_steps), s));
    int st = step_run(c, latent, tb, B, lat_f, H8, W8, nullptr, nullptr, kv_cache, w, vel, wsb, y, s,
                      q8buf);
    if (st) return st;
    WAN_TRY(launch_euler(latent, vel, B, c.in_ch, c.out_ch, plane, dt, guided, scale, s));
  }
  return WAN_OK;
}

// ---- the block without a caller workspace
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
char *scratch_dev[MAX_DEVICES];   // device address of `scratch` per device ordinal

// the current device's scratch address (looked up on the first call on that
// device, with the device current); nullptr when the lookup fails
char *scratch_base() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_dev[dev] = static_cast<char *>(p);
  }
  return scratch_dev[dev];
}

}  // namespace

extern "C" {

const char *wan_status_str(int st) {
  switch (st) {
    case WAN_OK: return "ok";
    case WAN_ERR_NULL: return "a required pointer is NULL";
    case WAN_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case WAN_ERR_DTYPE: return "unsupported dtype";
    case WAN_ERR_WORKSPACE: return "workspace too small";
    case WAN_ERR_CONFIG: return "I2V inputs inconsistent with the configuration";
    case WAN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t wan_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int H8, int W8) {
  if (check_cfg(cfg) != WAN_OK) return 0;
  if (H8 <= 0 || W8 <= 0 || H8 % 2 || W8 % 2) return 0;
  if (check_dims(*cfg, B, lat_f, H8 / 2, W8 / 2) != WAN_OK) return 0;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  return make_layout(*cfg, B, L, true).total;
}

int wan_tmlp_fwd(const wan_cfg_t *cfg, const float *t, int B, const wan_tmlp_weights_t *w,
                 float *mod, void *ws, size_t ws_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!t || !w || !mod || !ws || !w->w1 || !w->b1 || !w->w2 || !w->b2) return WAN_ERR_NULL;
  if (B <= 0 || B > 8) return WAN_ERR_SHAPE;
  const size_t need = (size_t)B * (cfg->dim + cfg->freq_dim) * 4;
  if (ws_bytes < need) return WAN_ERR_WORKSPACE;
  WAN_TRY(launch_tmlp(t, B, cfg->freq_dim, cfg->dim, w->w1, w->b1, w->w2, w->b2, (float *)ws, mod,
                      cfg->dtype == WAN_F32, S(stream)));
  return WAN_OK;
}

int wan_dit_block_fwd(const wan_cfg_t *cfg, float *x, int B, int lat_f, int Hp, int Wp,
                      const float *mod, const wan_block_weights_t *w, const void *ctx,
                      const void *img_ctx, void *ws, size_t ws_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!x || !mod || !ctx || !ws) return WAN_ERR_NULL;
  if ((st = check_dims(*cfg, B, lat_f, Hp, Wp))) return st;
  if ((st = check_block_weights(*cfg, w))) return st;
  if ((cfg->img_len > 0) != (img_ctx != nullptr)) return WAN_ERR_CONFIG;
  const long L = (long)lat_f * Hp * Wp;
  Layout y = make_layout(*cfg, B, L, false);
  if (ws_bytes < y.total) return WAN_ERR_WORKSPACE;
  return block_run(*cfg, x, B, L, mod, *w, ctx, img_ctx, nullptr, (char *)ws, y, S(stream));
}

size_t wan_dit_block_noalloc_bytes(const wan_cfg_t *cfg, int B, int lat_f, int Hp, int Wp) {
  if (check_cfg(cfg) != WAN_OK || check_dims(*cfg, B, lat_f, Hp, Wp) != WAN_OK) return 0;
  return make_layout(*cfg, B, (long)lat_f * Hp * Wp, false).total;
}

int wan_dit_block_fwd_noalloc(const wan_cfg_t *cfg, float *x, int B, int lat_f, int Hp, int Wp,
                              const float *mod, const wan_block_weights_t *w, const void *ctx,
                              const void *img_ctx, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!x || !mod || !ctx) return WAN_ERR_NULL;
  if ((st = check_dims(*cfg, B, lat_f, Hp, Wp))) return st;
  if ((st = check_block_weights(*cfg, w))) return st;
  if ((cfg->img_len > 0) != (img_ctx != nullptr)) return WAN_ERR_CONFIG;
  const long L = (long)lat_f * Hp * Wp;
  Layout y = make_layout(*cfg, B, L, false);
  if (y.total > WAN_NOALLOC_SCRATCH_BYTES) return WAN_ERR_WORKSPACE;
  char *ws = scratch_base();
  if (!ws) return WAN_ERR_HIP;
  return block_run(*cfg, x, B, L, mod, *w, ctx, img_ctx, nullptr, ws, y, S(stream));
}

int wan_dit_step_fwd(const wan_cfg_t *cfg, const float *latent, const float *t, int B, int lat_f,
                     int H8, int W8, const void *ctx, const void *clip_feat,
                     const wan_model_weights_t *w, float *out, void *ws, size_t ws_bytes,
                     void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!latent || !t || !ctx || !w || !out || !ws) return WAN_ERR_NULL;
  if ((st = check_step_dims(*cfg, B, lat_f, H8, W8))) return st;
  const bool i2v = cfg->img_len > 0;
  if ((st = check_model_weights(*cfg, w, i2v))) return st;
  if (i2v != (clip_feat != nullptr)) return WAN_ERR_CONFIG;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  Layout y = make_layout(*cfg, B, L, true);
  if (ws_bytes < y.total) return WAN_ERR_WORKSPACE;
  return step_run(*cfg, latent, t, B, lat_f, H8, W8, ctx, clip_feat, nullptr, *w, out, (char *)ws,
                  y, S(stream));
}

size_t wan_kv_cache_bytes(const wan_cfg_t *cfg, int B) {
  if (check_cfg(cfg) != WAN_OK || B <= 0 || B > 8) return 0;
  return kv_layout(*cfg, B).per_block * (size_t)cfg->n_blocks;
}

int wan_kv_cache_fwd(const wan_cfg_t *cfg, int B, const void *ctx, const void *clip_feat,
                     const wan_model_weights_t *w, void *cache, size_t cache_bytes, void *ws,
                     size_t ws_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!ctx || !w || (!cache && cfg->n_blocks > 0)) return WAN_ERR_NULL;
  if (B <= 0 || B > 8) return WAN_ERR_SHAPE;
  const bool i2v = cfg->img_len > 0;
  if ((st = check_model_weights(*cfg, w, i2v))) return st;
  if (i2v != (clip_feat != nullptr)) return WAN_ERR_CONFIG;
  const KvLayout kl = kv_layout(*cfg, B);
  if (cache_bytes < kl.per_block * (size_t)cfg->n_blocks) return WAN_ERR_WORKSPACE;
  const size_t es = cfg->dtype == WAN_F32 ? 4 : 2;
  const size_t img_bytes = up((size_t)B * cfg->img_len * cfg->dim * es, ALIGN);
  if (i2v && (!ws || ws_bytes < 3 * img_bytes)) return i2v && !ws ? WAN_ERR_NULL : WAN_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  char *wsb = (char *)ws;
  const void *img = nullptr;
  if (i2v) {
    if ((st = image_context(*cfg, B, clip_feat, *w, wsb, wsb + img_bytes, wsb + 2 * img_bytes, s)))
      return st;
    img = wsb + 2 * img_bytes;
  }
  for (int i = 0; i < cfg->n_blocks; ++i) {
    char *base = (char *)cache + (size_t)i * kl.per_block;
    const wan_block_weights_t &bw = w->blocks[i];
    if ((st = kv_project(*cfg, B, cfg->text_len, ctx, bw.ca_wkv, bw.ca_bkv, base + kl.kc,
                         base + kl.vtc, rup(cfg->text_len, 64), s)))
      return st;
    if (i2v && (st = kv_project(*cfg, B, cfg->img_len, img, bw.ca_wkv_img, bw.ca_bkv_img,
                                base + kl.ki, base + kl.vti, rup(cfg->img_len, 64), s)))
      return st;
  }
  return WAN_OK;
}

int wan_dit_step_cached_fwd(const wan_cfg_t *cfg, const float *latent, const float *t, int B,
                            int lat_f, int H8, int W8, const void *kv_cache, size_t cache_bytes,
                            const wan_model_weights_t *w, float *out, void *ws, size_t ws_bytes,
                            void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!latent || !t || !w || !out || !ws || (!kv_cache && cfg->n_blocks > 0)) return WAN_ERR_NULL;
  if ((st = check_step_dims(*cfg, B, lat_f, H8, W8))) return st;
  if ((st = check_model_weights(*cfg, w, false))) return st;
  if (cache_bytes < kv_layout(*cfg, B).per_block * (size_t)cfg->n_blocks) return WAN_ERR_WORKSPACE;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  Layout y = make_layout(*cfg, B, L, true);
  if (ws_bytes < y.total) return WAN_ERR_WORKSPACE;
  return step_run(*cfg, latent, t, B, lat_f, H8, W8, nullptr, nullptr, (const char *)kv_cache, *w,
                  out, (char *)ws, y, S(stream));
}

int wan_euler_fwd(float *latent, const float *vel, int B, int in_ch, int out_ch, int lat_f, int H8,
                  int W8, float dt, int guided, float scale, void *stream) {
  if (!latent || !vel) return WAN_ERR_NULL;
  if (B <= 0 || B > 8 || out_ch <= 0 || in_ch < out_ch || lat_f <= 0 || H8 <= 0 || W8 <= 0)
    return WAN_ERR_SHAPE;
  if (guided && B != 2) return WAN_ERR_SHAPE;
  if (!isfinite(dt) || !isfinite(scale)) return WAN_ERR_SHAPE;
  const long plane = (long)lat_f * H8 * W8;
  if ((long)B * in_ch * plane > (1L << 31)) return WAN_ERR_SHAPE;
  WAN_TRY(launch_euler(latent, vel, B, in_ch, out_ch, plane, dt, guided, scale, S(stream)));
  return WAN_OK;
}

size_t wan_sample_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int H8, int W8) {
  if (check_cfg(cfg) != WAN_OK || check_step_dims(*cfg, B, lat_f, H8, W8) != WAN_OK) return 0;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  size_t t_off, v_off;
  return sample_extra(B, cfg->out_ch, (long)lat_f * H8 * W8, &t_off, &v_off,
                      make_layout(*cfg, B, L, true).total);
}

int wan_sample_fwd(const wan_cfg_t *cfg, float *latent, int B, int lat_f, int H8, int W8,
                   int n_steps, int guided, float scale, const void *kv_cache, size_t cache_bytes,
                   const wan_model_weights_t *w, void *ws, size_t ws_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (!latent || !w || !ws || (!kv_cache && cfg->n_blocks > 0)) return WAN_ERR_NULL;
  if ((st = check_step_dims(*cfg, B, lat_f, H8, W8))) return st;
  if (n_steps <= 0 || (guided && B != 2) || !isfinite(scale)) return WAN_ERR_SHAPE;
  if (cfg->in_ch < cfg->out_ch) return WAN_ERR_SHAPE;
  if ((st = check_model_weights(*cfg, w, false))) return st;
  if (cache_bytes < kv_layout(*cfg, B).per_block * (size_t)cfg->n_blocks) return WAN_ERR_WORKSPACE;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  const long plane = (long)lat_f * H8 * W8;
  Layout y = make_layout(*cfg, B, L, true);
  size_t t_off, v_off;
  if (ws_bytes < sample_extra(B, cfg->out_ch, plane, &t_off, &v_off, y.total)) return WAN_ERR_WORKSPACE;
  return sample_run(*cfg, latent, B, lat_f, H8, W8, n_steps, guided, scale, (const char *)kv_cache, *w,
                    (char *)ws, y, t_off, v_off, S(stream));
}

int wan_i2v_mask(const uint8_t *frame_mask, int n_frames, int lat_f, int H8, int W8, float *out) {
  if (!frame_mask || !out) return WAN_ERR_NULL;
  if (n_frames <= 0 || lat_f <= 0 || H8 <= 0 || W8 <= 0) return WAN_ERR_SHAPE;
  if ((n_frames - 1) % 4 || (n_frames - 1) / 4 + 1 != lat_f) return WAN_ERR_SHAPE;
  const long plane = (long)H8 * W8;
  for (int ch = 0; ch < 4; ++ch)
    for (int f = 0; f < lat_f; ++f) {
      // extended sequence: frame 0 four times, then frames 1..n-1; group f, member ch
      const int e = f * 4 + ch;
      const int src = e < 4 ? 0 : e - 3;
      const float v = frame_mask[src] ? 1.0f : 0.0f;
      float *p = out + ((long)ch * lat_f + f) * plane;
      for (long i = 0; i < plane; ++i) p[i] = v;
    }
  return WAN_OK;
}

int wan_attention_fwd(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv,
                      int vt_bstride, void *o, int ldo, int B, int H, int Lq, int Lk, int q_scaled,
                      void *stream) {
  if (!q || !k || !vt || !o) return WAN_ERR_NULL;
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0) return WAN_ERR_SHAPE;
  if (ldq < (long)H * 128 || ldk < (long)H * 128 || ldo < (long)H * 128 || ldq % 8 || ldk % 8 || ldo % 4)
    return WAN_ERR_SHAPE;
  if (ldv % 8 || vt_bstride % 8 || vt_bstride < rup(Lk, 64) || (long)ldv < (long)B * vt_bstride)
    return WAN_ERR_SHAPE;
  AttnDesc a = attn(q, ldq, k, ldk, vt, ldv, vt_bstride, o, ldo, B, H, Lq, Lk, 128, 0, q_scaled != 0);
  WAN_TRY(launch_attention(a, S(stream)));
  return WAN_OK;
}


size_t wan_attention_8bit_workspace_bytes(int B, int H, int Lq, int Lk) {
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || !attn8_fits(B, H, Lq, Lk)) return 0;
  size_t off[7];
  attn8_offsets(B, H, Lq, Lk, off);
  return off[6];
}

int wan_attention_8bit_quantize(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv,
                                int vt_bstride, int B, int H, int Lq, int Lk, void *q8, float *qs, void *k8,
                                float *ks, void *v8t, float *vs, void *stream) {
  if (!q || !k || !vt || !q8 || !qs || !k8 || !ks || !v8t || !vs) return WAN_ERR_NULL;
  const int st = attn8_check_inputs(ldq, ldk, ldv, vt_bstride, B, H, Lq, Lk);
  if (st != WAN_OK) return st;
  WAN_TRY(launch_quant_attn8(attn8_quant(q, ldq, k, ldk, vt, ldv, vt_bstride, B, H, Lq, Lk, q8, qs, k8, ks,
                                         v8t, vs), S(stream)));
  return WAN_OK;
}

int wan_attention_8bit_q_fwd(const void *q8, const float *qs, const void *k8, const float *ks, const void *v8t,
                             const float *vs, void *o, int ldo, int B, int H, int Lq, int Lk, int q_scaled,
                             void *stream) {
  if (!q8 || !qs || !k8 || !ks || !v8t || !vs || !o) return WAN_ERR_NULL;
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || ldo < (long)H * 128 || ldo % 4) return WAN_ERR_SHAPE;
  if (!attn8_fits(B, H, Lq, Lk)) return WAN_ERR_SHAPE;
  WAN_TRY(launch_attention8(attn8_desc(q8, qs, k8, ks, v8t, vs, o, ldo, B, H, Lq, Lk, q_scaled != 0), S(stream)));
  return WAN_OK;
}

int wan_attention_8bit_fwd(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv,
                           int vt_bstride, void *o, int ldo, int B, int H, int Lq, int Lk, int q_scaled,
                           void *ws, size_t ws_bytes, void *stream) {
  if (!q || !k || !vt || !o || !ws) return WAN_ERR_NULL;
  int st = attn8_check_inputs(ldq, ldk, ldv, vt_bstride, B, H, Lq, Lk);
  if (st != WAN_OK) return st;
  if (ldo < (long)H * 128 || ldo % 4) return WAN_ERR_SHAPE;
  size_t off[7];
  attn8_offsets(B, H, Lq, Lk, off);
  if (ws_bytes < off[6]) return WAN_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  float *qs = (float *)(w + off[1]), *ks = (float *)(w + off[3]), *vs = (float *)(w + off[5]);
  WAN_TRY(launch_quant_attn8(attn8_quant(q, ldq, k, ldk, vt, ldv, vt_bstride, B, H, Lq, Lk, w + off[0], qs,
                                         w + off[2], ks, w + off[4], vs), S(stream)));
  WAN_TRY(launch_attention8(attn8_desc(w + off[0], qs, w + off[2], ks, w + off[4], vs, o, ldo, B, H, Lq, Lk,
                                       q_scaled != 0), S(stream)));
  return WAN_OK;
}

int wan_quantize_rows_fp8(const void *x, int M, int K, int ldx, void *q, int ldq, float *scale,
                          void *stream) {
  if (!x || !q || !scale) return WAN_ERR_NULL;
  if (M <= 0 || K <= 0 || K % 8 || ldx < K || ldq < K || ldx % 8 || ldq % 8) return WAN_ERR_SHAPE;
  WAN_TRY(launch_quant_rows_fp8(x, M, K, ldx, q, ldq, scale, S(stream)));
  return WAN_OK;
}

int wan_quantize_tensor_fp8(const void *w, long n, void *q, float *scale, void *ws, size_t ws_bytes,
                            void *stream) {
  if (!w || !q || !scale || !ws) return WAN_ERR_NULL;
  if (n <= 0 || n % 8) return WAN_ERR_SHAPE;
  if (ws_bytes < 4) return WAN_ERR_WORKSPACE;
  WAN_TRY(launch_quant_tensor_fp8(w, n, q, scale, (unsigned *)ws, S(stream)));
  return WAN_OK;
}

int wan_linear_fp8_fwd(const void *xq, const float *x_scale, const void *wq, const float *w_scale,
                       const void *b, void *y, int M, int N, int K, int mode, void *stream) {
  if (!xq || !x_scale || !wq || !w_scale || !y) return WAN_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || K % 64) return WAN_ERR_SHAPE;
  int kind = mode == 0 ? OUT_BF16 : mode == 1 ? OUT_F32 : mode == 2 ? OUT_GELU : -1;
  if (kind < 0) return WAN_ERR_CONFIG;
  GemmDesc g = gemm(xq, K, wq, K, M, N, K, b, kind, y, N, 0);
  g.fp8 = 1;
  g.a_scale = x_scale;
  g.b_scale = w_scale;
  g.a_per_row = 1;
  WAN_TRY(launch_gemm(g, S(stream)));
  return WAN_OK;
}

size_t wan_block_fp8_bytes(const wan_cfg_t *cfg) {
  if (check_cfg(cfg) != WAN_OK || cfg->dtype != WAN_BF16) return 0;
  return fp8_layout(*cfg).total;
}

int wan_quantize_block_fp8(const wan_cfg_t *cfg, const wan_block_weights_t *w, void *qbuf,
                           size_t qbuf_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (!w || !qbuf) return WAN_ERR_NULL;
  const void *src[6] = {w->sa_wqkv, w->sa_wo, w->ca_wq, w->ca_wo, w->ffn_w1, w->ffn_w2};
  for (const void *p : src)
    if (!p) return WAN_ERR_NULL;
  const Fp8Layout q = fp8_layout(*cfg);
  if (qbuf_bytes < q.total) return WAN_ERR_WORKSPACE;
  if ((uintptr_t)qbuf % ALIGN) return WAN_ERR_SHAPE;
  char *b = (char *)qbuf;
  for (int i = 0; i < 6; ++i)
    WAN_TRY(launch_quant_tensor_fp8(src[i], q.n[i], b + q.w[i], (float *)(b + q.sc) + i,
                                    (unsigned *)(b + q.amax) + i, S(stream)));
  return WAN_OK;
}

size_t wan_block_fp8_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int Hp, int Wp) {
  if (check_cfg(cfg) != WAN_OK || cfg->dtype != WAN_BF16) return 0;
  if (check_dims(*cfg, B, lat_f, Hp, Wp) != WAN_OK) return 0;
  return make_layout(*cfg, B, (long)lat_f * Hp * Wp, false, true).total;
}

int wan_dit_block_fp8_fwd(const wan_cfg_t *cfg, float *x, int B, int lat_f, int Hp, int Wp,
                          const float *mod, const wan_block_weights_t *w, const void *qbuf,
                          const void *ctx, const void *img_ctx, void *ws, size_t ws_bytes,
                          void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (!x || !mod || !ctx || !ws || !qbuf) return WAN_ERR_NULL;
  if ((uintptr_t)qbuf % ALIGN) return WAN_ERR_SHAPE;
  if ((st = check_dims(*cfg, B, lat_f, Hp, Wp))) return st;
  if ((st = check_block_weights(*cfg, w, true))) return st;
  if ((cfg->img_len > 0) != (img_ctx != nullptr)) return WAN_ERR_CONFIG;
  const long L = (long)lat_f * Hp * Wp;
  // one sample's FP8 operands below 2 GiB (larger GEMMs are split at samples)
  if (L * (cfg->ffn > cfg->dim ? cfg->ffn : cfg->dim) >= (1L << 31)) return WAN_ERR_SHAPE;
  Layout y = make_layout(*cfg, B, L, false, true);
  if (ws_bytes < y.total) return WAN_ERR_WORKSPACE;
  const Fp8Layout ql = fp8_layout(*cfg);
  const char *qb = (const char *)qbuf;
  Fp8Ptrs q8;
  for (int i = 0; i < 6; ++i) q8.w[i] = (const uint8_t *)(qb + ql.w[i]);
  q8.sc = (const float *)(qb + ql.sc);
  q8.aq = (uint8_t *)ws + y.aq;
  q8.as = (float *)((char *)ws + y.as);
  return block_run(*cfg, x, B, L, mod, *w, ctx, img_ctx, nullptr, (char *)ws, y, S(stream), &q8);
}

size_t wan_model_fp8_bytes(const wan_cfg_t *cfg) {
  if (check_cfg(cfg) != WAN_OK || cfg->dtype != WAN_BF16) return 0;
  return fp8_layout(*cfg).total * (size_t)cfg->n_blocks;
}

int wan_quantize_model_fp8(const wan_cfg_t *cfg, const wan_model_weights_t *w, void *qbuf,
                           size_t qbuf_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (!w || (!qbuf && cfg->n_blocks > 0) || (cfg->n_blocks > 0 && !w->blocks)) return WAN_ERR_NULL;
  const size_t per = fp8_layout(*cfg).total;
  if (qbuf_bytes < per * (size_t)cfg->n_blocks) return WAN_ERR_WORKSPACE;
  for (int i = 0; i < cfg->n_blocks; ++i)
    if ((st = wan_quantize_block_fp8(cfg, &w->blocks[i], (char *)qbuf + (size_t)i * per, per, stream)))
      return st;
  return WAN_OK;
}

size_t wan_fp8_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int H8, int W8, int sampler) {
  if (check_cfg(cfg) != WAN_OK || cfg->dtype != WAN_BF16) return 0;
  if (check_step_dims(*cfg, B, lat_f, H8, W8) != WAN_OK) return 0;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  const size_t base = make_layout(*cfg, B, L, true, true).total;
  if (!sampler) return base;
  size_t t_off, v_off;
  return sample_extra(B, cfg->out_ch, (long)lat_f * H8 * W8, &t_off, &v_off, base);
}

int wan_dit_step_fp8_fwd(const wan_cfg_t *cfg, const float *latent, const float *t, int B, int lat_f,
                         int H8, int W8, const void *ctx, const void *clip_feat,
                         const wan_model_weights_t *w, const void *qbuf, float *out, void *ws,
                         size_t ws_bytes, void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (!latent || !t || !ctx || !w || !out || !ws || (!qbuf && cfg->n_blocks > 0)) return WAN_ERR_NULL;
  if ((uintptr_t)qbuf % ALIGN) return WAN_ERR_SHAPE;
  if ((st = check_step_dims(*cfg, B, lat_f, H8, W8))) return st;
  const bool i2v = cfg->img_len > 0;
  if ((st = check_model_weights(*cfg, w, i2v, true))) return st;
  if (i2v != (clip_feat != nullptr)) return WAN_ERR_CONFIG;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  if (L * (cfg->ffn > cfg->dim ? cfg->ffn : cfg->dim) >= (1L << 31)) return WAN_ERR_SHAPE;
  Layout y = make_layout(*cfg, B, L, true, true);
  if (ws_bytes < y.total) return WAN_ERR_WORKSPACE;
  return step_run(*cfg, latent, t, B, lat_f, H8, W8, ctx, clip_feat, nullptr, *w, out, (char *)ws, y,
                  S(stream), (const char *)qbuf);
}

int wan_sample_fp8_fwd(const wan_cfg_t *cfg, float *latent, int B, int lat_f, int H8, int W8,
                       int n_steps, int guided, float scale, const void *kv_cache, size_t cache_bytes,
                       const wan_model_weights_t *w, const void *qbuf, void *ws, size_t ws_bytes,
                       void *stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != WAN_BF16) return WAN_ERR_DTYPE;
  if (!latent || !w || !ws || ((!kv_cache || !qbuf) && cfg->n_blocks > 0)) return WAN_ERR_NULL;
  if ((uintptr_t)qbuf % ALIGN) return WAN_ERR_SHAPE;
  if ((st = check_step_dims(*cfg, B, lat_f, H8, W8))) return st;
  if (n_steps <= 0 || (guided && B != 2) || !isfinite(scale)) return WAN_ERR_SHAPE;
  if (cfg->in_ch < cfg->out_ch) return WAN_ERR_SHAPE;
  if ((st = check_model_weights(*cfg, w, false, true))) return st;
  if (cache_bytes < kv_layout(*cfg, B).per_block * (size_t)cfg->n_blocks) return WAN_ERR_WORKSPACE;
  const long L = (long)lat_f * (H8 / 2) * (W8 / 2);
  if (L * (cfg->ffn > cfg->dim ? cfg->ffn : cfg->dim) >= (1L << 31)) return WAN_ERR_SHAPE;
  const long plane = (long)lat_f * H8 * W8;
  Layout y = make_layout(*cfg, B, L, true, true);
  size_t t_off, v_off;
  if (ws_bytes < sample_extra(B, cfg->out_ch, plane, &t_off, &v_off, y.total)) return WAN_ERR_WORKSPACE;
  return sample_run(*cfg, latent, B, lat_f, H8, W8, n_steps, guided, scale, (const char *)kv_cache, *w,
                    (char *)ws, y, t_off, v_off, S(stream), (const char *)qbuf);
}

int wan_set_attention_events(void *start, void *stop) {
  if ((start == nullptr) != (stop == nullptr)) return WAN_ERR_NULL;
  att_ev_start = static_cast<hipEvent_t>(start);
  att_ev_stop = static_cast<hipEvent_t>(stop);
  return WAN_OK;
}

int wan_ln_modulate_fwd(const float *x, int B, int L, int d, const float *mod, int branch, float eps,
                        void *h, void *stream) {
  if (!x || !h) return WAN_ERR_NULL;
  if (B <= 0 || B > 8 || L <= 0 || d <= 0 || (long)B * L > (1L << 30)) return WAN_ERR_SHAPE;
  if (!(eps > 0.f) || !isfinite(eps)) return WAN_ERR_SHAPE;
  if (mod && branch != 0 && branch != 1) return WAN_ERR_CONFIG;
  const int shift_off = branch ? 3 * d : 0, scale_off = branch ? 4 * d : d;
  WAN_TRY(launch_ln_mod(x, B * L, L, d, mod, 6L * d, shift_off, scale_off, mod != nullptr, eps, h, 0,
                        S(stream)));
  return WAN_OK;
}

int wan_linear_fwd(const void *x, const void *w, const void *b, void *y, int M, int N, int K,
                   int mode, void *stream) {
  if (!x || !w || !y) return WAN_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || K % 64) return WAN_ERR_SHAPE;
  int kind = mode == 0 ? OUT_BF16 : mode == 1 ? OUT_F32 : mode == 2 ? OUT_GELU : -1;
  if (kind < 0) return WAN_ERR_CONFIG;
  WAN_TRY(launch_gemm(gemm(x, K, w, K, M, N, K, b, kind, y, N, 0), S(stream)));
  return WAN_OK;
}

}  // extern "C"
