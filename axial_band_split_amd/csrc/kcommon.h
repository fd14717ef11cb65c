// Device-side types shared by the kernels of the core: element types, 16-byte MFMA operand
// fragments, the gfx950 matrix-core instructions used, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mbr {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each lane feeds 16 bytes of A and 16 bytes of B per matrix-core step:
//   f16 / bf16: v_mfma_f32_16x16x32 (8 elements per lane, K = 32 per step)
//   f32:        4 x v_mfma_f32_16x16x4f32 (4 elements per lane, K = 16 per step)
// Lane l holds row (A) / column (B) l % 16 and K elements EPF*(l/16) .. EPF*(l/16)+EPF-1.  The
// accumulator C (16x16) holds, in lane l, column l % 16 and rows 4*(l/16) .. 4*(l/16)+3.
template <typename T> struct Frag;
template <> struct Frag<f16> { typedef f16x8 type; typedef f16x4 half_type; static constexpr int EPF = 8; };
template <> struct Frag<bf16> { typedef bf16x8 type; typedef bf16x4 half_type; static constexpr int EPF = 8; };
template <> struct Frag<float> { typedef f32x4 type; typedef float half_type; static constexpr int EPF = 4; };

// Four elements of T in one vector register group (8 or 16 bytes).
template <typename T> struct Vec4;
template <> struct Vec4<f16> { typedef f16x4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

__device__ __forceinline__ void mma(f32x4& c, const f16x8& a, const f16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32: the four instructions take the lane's elements 0..3 in turn; lane group g = l/16 is the
// instruction's own k index, so instruction j covers k = 4*g + j of the 16 and all four together
// cover every k once (the k order of a sum is free).
__device__ __forceinline__ void mma(f32x4& c, const f32x4& a, const f32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T cvt(float x) { return (T)x; }
template <typename T> __device__ __forceinline__ float tof(T x) { return (float)x; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// sigma(x) = 1 / (1 + 2^(-x log2 e)) with the hardware exp2 and reciprocal (about 2 ulp; 0 and 1
// at the extremes, where the exponential is inf or 0)
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}
// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2), t = 1 / (1 + p z), z >= 0, with
// |error| <= 1.5e-7; odd in z.  One reciprocal, five FMAs and one exponential.
__device__ __forceinline__ float erf_as(float x) {
  const float z = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  return copysignf(fmaf(-p, e, 1.0f), x);
}
// tanh x = 1 - 2 / (e^{2x} + 1): one exponential and one reciprocal (absolute error a few 1e-7,
// far below the 16-bit rounding of the values it feeds; +-1 at the extremes, where e^{2x} is inf or 0).
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * 2.8853900817779268f));
}
// GELU with the error function (x * Phi(x)), as the feed-forward of the core uses it.
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f)); }
// Twice the GELU for values that are then rounded to 16 bits: 2 x Phi(x) = x + |x| (1 - 2 Q(|x|)),
// Q the upper tail of the standard normal distribution, with 2 Q(a) = 2^p(a) for a cubic p without
// constant term (so 2 Q(0) = 1 exactly); its three coefficients are a minimax fit of the weighted
// error max(a, 1) |2^(p(a) - 1) - Q(a)| over [0, 10] (gelu_tail_fit.py beside this file).  All three
// are negative, so p falls for every a >= 0 and the tail goes to zero.  The GELU is within 1.3e-4
// absolute and 1.3e-4 |x| of the erf GELU everywhere, below a 16-bit rounding (a relative step of
// 4.9e-4 in fp16); for large negative x the sum cancels to within 1e-7 absolute.  Four vector
// instructions and one exp2, against about ten and two transcendental ones for gelu_erf.
__device__ __forceinline__ float gelu2_tail(float x) {
  const float a = fabsf(x);
  float p = fmaf(-0.030005693f, a, -0.48125008f);
  p = fmaf(p, a, -1.1454322f);
  p *= a;
  return fmaf(a, 1.0f - __builtin_amdgcn_exp2f(p), x);
}

constexpr float kNormEps = 1e-12f;

// A raw buffer over [base, base + bytes) for the loads below (bytes < 2^31; reads past the end
// return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// The same over a base and size the caller knows to be wave-uniform but the compiler may not (values
// read from memory): taken from the first lane, so the descriptor lives in scalar registers and
// every load through it is one instruction (a descriptor in vector registers costs a loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p), hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return buffer_rsrc((const void*)(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}
// 16 bytes per lane from buffer offset voff (per lane) + soff (uniform) into LDS at
// lds_wave_base + 16 * lane.  The buffer form of the LDS load and not the global one: with a
// FLAT-encoded load to LDS in flight the compiler must assume LDS reads complete out of order and
// waits for every one of them (lgkmcnt(0)) before any use, which serialises pipelined reads.
__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t rs, int voff, int soff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff, 0, 0);
}

}  // namespace mbr
