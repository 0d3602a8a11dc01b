// Device-side types and helpers shared by the gfx950 kernels of libwandit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define WAN_DEV __device__ __forceinline__

// round-to-nearest-even float -> bf16 (gfx950 has it in hardware)
WAN_DEV bf16 f2bf(float x) { return (bf16)x; }
WAN_DEV float bf2f(bf16 x) { return (float)x; }

template <typename T> WAN_DEV float to_f(T v);
template <> WAN_DEV float to_f<float>(float v) { return v; }
template <> WAN_DEV float to_f<bf16>(bf16 v) { return (float)v; }

template <typename T> WAN_DEV T from_f(float v);
template <> WAN_DEV float from_f<float>(float v) { return v; }
template <> WAN_DEV bf16 from_f<bf16>(float v) { return (bf16)v; }

// 16-byte global load / store helpers
WAN_DEV uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
WAN_DEV void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

WAN_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
WAN_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// tanh-approximated GELU, 0.5 u (1 + tanh(y)) with y = sqrt(2/pi)(u + 0.044715 u^3),
// written as u * sigmoid(2y) = u / (1 + 2^(-2 y log2 e)): one v_exp_f32 and
// one v_rcp_f32 (each about 1 ulp).  For large |u| the exponential goes to 0
// or +inf and the reciprocal to 1 or 0, giving u and 0 without a clamp.
WAN_DEV float gelu_tanh(float u) {
  const float a = -2.0f * 1.4426950408889634f * 0.7978845608028654f;   // -2 log2(e) sqrt(2/pi)
  const float b = a * 0.044715f;
  const float z = u * fmaf(b, u * u, a);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

WAN_DEV float silu(float z) { return z / (1.0f + __expf(-z)); }

// XCD-aware block index: the hardware deals workgroups round-robin over the
// 8 XCDs; remap so that each XCD receives a contiguous range of logical
// tiles (neighbouring tiles then share that XCD's L2).
WAN_DEV int xcd_remap(int bid, int nblocks) {
  const int nx = 8;
  int per = nblocks / nx;           // blocks every XCD gets
  int rem = nblocks - per * nx;     // the first `rem` XCDs get one more
  int x = bid % nx, i = bid / nx;
  if (i >= per) return per * nx + x;  // tail round (x < rem): keep at the end
  (void)rem;
  return x * per + i;
}
