// Launch interface of the attention kernels of libwandit (internal).
#pragma once
#include <hip/hip_runtime.h>

namespace wan {

// Attention O = softmax(Q K^T * scale) V for every (batch, head); hd = 128, bf16.
struct AttnDesc {
  const void *q; long ldq;     // [B*Lq, ldq], head h at column h*hd
  const void *k; long ldk;     // [B*Lk, ldk]
  const void *vt; long ldv; long vt_bstride;  // [H*hd, ldv], batch b at column b*vt_bstride
  void *o; long ldo;           // [B*Lq, ldo]
  int B, H, Lq, Lk, hd;
  float scale;                 // 1/sqrt(hd)
  int out_mode;                // 0: o = O (bf16); 1: acc32 = O; 2: o = acc32 + O
  float *acc32;                // [B*Lq, H*hd] float32 partial (modes 1, 2)
  int f32;                     // float32 path (generic kernel): v given untransposed in `vt`
  int q_scaled;                // bf16 path: q already multiplied by scale * log2(e)
};

hipError_t launch_attention(const AttnDesc &a, hipStream_t s);

}  // namespace wan
