// Device helpers shared by the fp8bs kernels (gfx950 only).
//
// e4m3 "fn" format: 1 sign, 4 exponent, 3 mantissa bits, largest finite 448
// (the fourth page, "Converting DeepSeek-V4's Indexer GEMM from FP32 to bf16",
// section "Assumptions and Their Validity"; 448 as the divisor of the dynamic
// scale in TensorRT-LLM PR "Size the per-tensor FP8 dynamic-quant amax grid to
// the input", section "Correctness").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

constexpr float kE4m3Max = 448.0f;

// Scales at or above this value take the three-operation quotient below; a
// smaller nonzero scale (block maximum under about 2.4e-17) divides with the
// full IEEE sequence instead, so that every intermediate of the fast quotient
// stays a normal binary32 number.
constexpr float kFastScaleMin = 0x1p-64f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Correctly rounded x / s from r = fl32(1 / s): q0 = x*r, one remainder by
// FMA and one correction by FMA (Markstein's correction step; P. Markstein,
// IBM J. Res. Dev. 34(1), 1990). The remainder is taken negated,
// e' = q0*s - x, and the correction is q0 - e'*r: the same bits as
// x - q0*s and q0 + e*r for every nonzero x (round-to-nearest is symmetric),
// and the sign of a zero x survives (-0 stays -0, which encodes to 0x80).
// For bf16 x and s = fl32(amax / 448) with amax bf16, the quotient's
// significand depends only on the significands of x and amax; the result
// equals the IEEE quotient for every such pair (checked exhaustively over all
// 128 x 128 significand pairs and 15 binades of x below amax, on the CPU and
// through the kernels on the GPU). Requires s >= kFastScaleMin.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
#pragma clang fp contract(off)
  const float q0 = x * r;
  const float en = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-en, r, q0);
}

// IEEE binary32 division (the compiler's correctly rounded sequence).
__device__ __forceinline__ float div_ieee(float x, float s) {
#pragma clang fp contract(off)
  return x / s;
}

// Four binary32 values -> four e4m3 codes in one dword (byte i = value i).
// Clamp to +-448 (v_med3), then the hardware conversion, which rounds to
// nearest even and keeps the sign of zero results.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4m3Max, kE4m3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4m3Max, kE4m3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4m3Max, kE4m3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4m3Max, kE4m3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// max over |bf16| of the two halves of a dword, as binary32 (exact)
__device__ __forceinline__ float absmax2(uint32_t w, float m) {
  return fmaxf(m, fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w))));
}

// DPP helpers: lanes exchange values inside rows of 16 without LDS.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i of each 8 reads lane 7-i
constexpr int kDppRowMirror = 0x140;   // lane i of each 16 reads lane 15-i

// max over each aligned group of 8 lanes (non-negative inputs)
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return v;
}

// max over the whole wave of 64 lanes (non-negative inputs); result in every lane
__device__ __forceinline__ float wave_max(float v) {
  v = group8_max(v);
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));                 // 16-lane rows
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// quantize the 8 bf16 of a uint4 with scale s (and r = 1/s on the fast path)
template <bool kFast>
__device__ __forceinline__ uint2 quant8(const uint4 v, float s, float r) {
  float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = kFast ? div_by_scale(f[i], s, r) : div_ieee(f[i], s);
  return make_uint2(pack4_e4m3(f[0], f[1], f[2], f[3]), pack4_e4m3(f[4], f[5], f[6], f[7]));
}

// One 1x128 block of bf16 held by an aligned group of 8 lanes, 16 elements
// a lane in two uint4 (v0, v1): amax over the group, s = fl32(amax / 448),
// the lane's 16 codes e4m3(clamp(x / s)) in o0, o1; an all-zero block gets
// scale 0 and codes 0x00. Returns s (and the block's amax in amax_out). The quotient takes the three-operation
// form unless some lane of the wave has a scale below kFastScaleMin (the
// ballot keeps the choice wave-uniform); lanes outside any block must have
// left the wave before the call.
__device__ __forceinline__ float quant_block_bf16(const uint4 v0, const uint4 v1, uint2& o0, uint2& o1,
                                                  float& amax_out) {
  float m = 0.0f;
  m = absmax2(v0.x, m); m = absmax2(v0.y, m); m = absmax2(v0.z, m); m = absmax2(v0.w, m);
  m = absmax2(v1.x, m); m = absmax2(v1.y, m); m = absmax2(v1.z, m); m = absmax2(v1.w, m);
  const float amax = group8_max(m);
  float s = div_ieee(amax, kE4m3Max);
  const bool fast = s >= kFastScaleMin;
  if (__builtin_expect(__ballot(!fast) == 0, 1)) {
    const float r = div_ieee(1.0f, s);
    o0 = quant8<true>(v0, s, r);
    o1 = quant8<true>(v1, s, r);
  } else {
    o0 = quant8<false>(v0, s, 0.0f);
    o1 = quant8<false>(v1, s, 0.0f);
  }
  if (amax == 0.0f) {
    s = 0.0f;
    o0 = make_uint2(0u, 0u);
    o1 = make_uint2(0u, 0u);
  }
  amax_out = amax;
  return s;
}
__device__ __forceinline__ float quant_block_bf16(const uint4 v0, const uint4 v1, uint2& o0, uint2& o1) {
  float amax;
  return quant_block_bf16(v0, v1, o0, o1, amax);
}

}  // namespace fp8bs
