// E4M3 quantisation helpers shared by the kernels that write FP8 activations
// ("Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)",
// section Infra / 推理优化: FP8 GEMM with per-token activation scales).
//
// Format: OCP E4M3 (v_cvt_pk_fp8_f32 on gfx950: round to nearest even, no
// saturation -- inputs are clamped to +-448 first).  A scale maps the largest
// magnitude to 448: inv = 448 / amax (correctly rounded float32 division),
// code = E4M3(clamp(x * inv)), stored scale = amax / 448 (x ~= code * scale);
// an all-zero row or tensor gets scale 1.
#pragma once
#include "common.hpp"

namespace wan {

WAN_DEV float inv_scale(float amax) { return amax > 0.f ? 448.0f / amax : 1.0f; }
WAN_DEV float deq_scale(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

// two floats -> two E4M3 bytes (low byte first)
WAN_DEV unsigned short pack2(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (unsigned short)(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFF);
}

// four floats -> four E4M3 bytes
WAN_DEV unsigned pack4(float a, float b, float c, float d) {
  return (unsigned)pack2(a, b) | ((unsigned)pack2(c, d) << 16);
}

// 8 bf16 -> 8 E4M3 bytes scaled by inv
WAN_DEV uint2 quant8(const uint4 &u, float inv) {
  const bf16 *e = reinterpret_cast<const bf16 *>(&u);
  uint2 r;
  r.x = pack4((float)e[0] * inv, (float)e[1] * inv, (float)e[2] * inv, (float)e[3] * inv);
  r.y = pack4((float)e[4] * inv, (float)e[5] * inv, (float)e[6] * inv, (float)e[7] * inv);
  return r;
}

WAN_DEV float amax8(const uint4 &u, float m) {
  const bf16 *e = reinterpret_cast<const bf16 *>(&u);
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)e[i]));
  return m;
}

}  // namespace wan
