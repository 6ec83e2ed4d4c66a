// Device helpers shared by the gfx950 kernels of libw8a8.so.
//
// Numerics follow the symmetric INT8 quantiser of the page "FP8 vs INT8
// quantisation for DeepSeek" (section 3.2.1, int8 branch) as used by the
// block-wise and channel-wise schemes of "DeepSeek R1 INT8 quantisation in
// SGLang" (section 2.3):  s = fp32(max(amax, 1e-10) / 127),
// q = rne(fp32(x / s)).  Everything here is compiled with -ffp-contract=off
// so that no multiply is silently fused with a following add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr float kEps = 1e-10f;          // amax floor: an all-zero group gets a finite scale
constexpr float kQMax = 127.0f;
// A quotient estimate y = fp32(x * fp32(1/s)) lies within 2.3e-5 of the
// correctly rounded fp32(x / s) whenever |x / s| <= 127.00002 (both carry at
// most 3 half-ulps of relative error at magnitude <= 127).  If y is farther
// than 2^-15 (3.05e-5) from every half-integer, both round to the same
// integer; otherwise the exact division decides.
constexpr float kTieGuard = 0.499969482421875f;   // 0.5 - 2^-15

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

// 8 values from a 16-byte chunk of bf16 or fp16.
template <bool FP16>
__device__ __forceinline__ void unpack8(const uint4& c, float* v) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (FP16) {
      v[2 * i] = h2f(w[i] & 0xffffu);
      v[2 * i + 1] = h2f(w[i] >> 16);
    } else {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

__device__ __forceinline__ float amax_n(const float* v, int n) {
  float a = 0.f;
  for (int i = 0; i < n; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
  return a;
}

// ---------------------------------------------------------------- quantiser
struct QScale {
  float s;   // the group scale, fp32(max(amax, eps) / 127)
  float r;   // fp32(1 / s): only used for the estimate, never stored
};

__device__ __forceinline__ QScale make_scale(float amax) {
  QScale q;
  q.s = fmaxf(amax, kEps) / kQMax;     // correctly rounded fp32 division
  q.r = 1.0f / q.s;
  return q;
}

// The group scale of the INT4 weight quantiser (the same quantiser with a
// 4-bit range): fp32(max(amax, eps) / 7).  quant_one's estimate-and-guard
// argument holds a fortiori for |x / s| <= 7.
__device__ __forceinline__ QScale make_scale4(float amax) {
  QScale q;
  q.s = fmaxf(amax, kEps) / 7.0f;      // correctly rounded fp32 division
  q.r = 1.0f / q.s;
  return q;
}

// rne(fp32(x / s)) as a float holding an integer in [-127, 127].
__device__ __forceinline__ float quant_one(float x, QScale sc) {
  float y = __fmul_rn(x, sc.r);
  float t = __builtin_rintf(y);
  float d = __builtin_fabsf(__fsub_rn(y, t));
  if (__builtin_expect(d > kTieGuard, 0)) t = __builtin_rintf(x / sc.s);
  return t;
}

// Pack the low bytes of four integer-valued floats (each in [-127, 127]).
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  uint32_t ia = (uint32_t)(int)a, ib = (uint32_t)(int)b;
  uint32_t ic = (uint32_t)(int)c, id = (uint32_t)(int)d;
  uint32_t lo = __builtin_amdgcn_perm(ib, ia, 0x0c0c0400u);   // [a, b, 0, 0]
  uint32_t hi = __builtin_amdgcn_perm(id, ic, 0x0c0c0400u);   // [c, d, 0, 0]
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);          // [a, b, c, d]
}

// ---------------------------------------------------------------- reductions
// Max over the 8 lanes of each half of a 16-lane DPP row.
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm [1,0,3,2]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm [2,3,0,1]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  return v;
}

// Max over the 16 lanes of each DPP row.
__device__ __forceinline__ float max16(float v) {
  v = max8(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));  // row_ror:8
  return v;
}

// Max over the whole 64-lane wave; the result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Block-wide max for a 256-thread workgroup (4 waves); every thread gets it.
__device__ __forceinline__ float block_max256(float v, float* red4) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red4[w] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
  return r;
}

}  // namespace w8
