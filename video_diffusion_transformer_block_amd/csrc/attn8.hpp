// Launch interface of the 8-bit attention kernels of libwandit (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

// Int8 / E4M3 copies of q, k and V^T for the 8-bit attention, with their
// scales; hd = 128, bf16 inputs laid out as for the bf16 attention.
struct Attn8Quant {
  const void *q; long ldq;                     // [B*Lq, ldq], head h at column h*128
  const void *k; long ldk;                     // [B*Lk, ldk]
  const void *vt; long ldv; long vt_bstride;   // [H*128, ldv]; columns Lk .. round_up(Lk, 64)-1 readable
  int B, H, Lq, Lk;
  void *q8; long ldq8; float *qs;              // [B*Lq, ldq8] Int8, [B*Lq, H]
  void *k8; long ldk8; float *ks;              // [B*Lk, ldk8] Int8, [B, H, ceil(Lk/64)]
  void *v8t; long ldv8; long v8_bstride;       // [H*128, ldv8] E4M3, batch b at column b*v8_bstride
  float *vs;                                   // [B, H*128]
};

hipError_t launch_quant_attn8(const Attn8Quant &z, hipStream_t s);

// 8-bit attention on those copies: o [B*Lq, ldo] bf16.
struct Attn8Desc {
  const int8_t *q8; long ldq8; const float *qs;
  const int8_t *k8; long ldk8; const float *ks;
  const uint8_t *v8t; long ldv8; long v8_bstride; const float *vs;
  void *o; long ldo;
  int B, H, Lq, Lk;
  float alpha;                                 // log2(e)/sqrt(128), or 1 for a pre-scaled q
};

hipError_t launch_attention8(const Attn8Desc &a, hipStream_t s);

}  // namespace wan
