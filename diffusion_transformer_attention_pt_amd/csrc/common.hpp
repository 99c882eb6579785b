// Device-side helpers shared by the PT-DiT attention-core kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptdit {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its 16-bit pattern (uint16_t) in memory.
__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// float -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> two packed bf16 (low half = a), software round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf2_sw(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

// Two floats -> two packed bf16 (low half = a) with the hardware converter
// (v_cvt_pk_bf16_f32, round to nearest even under the default mode).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// 2^x on the transcendental unit (v_exp_f32); inputs here are <= 0 and results
// below the fp32 normal range may flush to zero.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 r;
  r.x = pack_bf2(f[0], f[1]); r.y = pack_bf2(f[2], f[3]);
  r.z = pack_bf2(f[4], f[5]); r.w = pack_bf2(f[6], f[7]);
  return r;
}

// software-RNE variant, for results specified bit-for-bit (window averages)
__device__ __forceinline__ uint4 pack8_sw(const float* f) {
  uint4 r;
  r.x = pack_bf2_sw(f[0], f[1]); r.y = pack_bf2_sw(f[2], f[3]);
  r.z = pack_bf2_sw(f[4], f[5]); r.w = pack_bf2_sw(f[6], f[7]);
  return r;
}

// D(16x16, fp32) += A(16x16, bf16) * B(16x16, bf16): lane l supplies A row
// (l % 16), k = 4*(l / 16) .. +4 and B column (l % 16), the same k range; D as
// below.
__device__ __forceinline__ floatx4 mfma_bf16_k16(const uint2& a, const uint2& b, floatx4 c) {
  typedef short shortx4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b), c,
                                                   0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies A row (l % 16), k = 8*(l / 16) .. +8 and B column (l % 16),
// the same k range; it receives D rows 4*(l / 16) .. +4 of column (l % 16).
__device__ __forceinline__ floatx4 mfma_bf16(const uint4& a, const uint4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x4, fp32) * B(4x16, fp32).
// Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; output layout as above.
__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Load 8 consecutive elements starting at p as 8 bf16 (fp32 sources are
// rounded to nearest even).
__device__ __forceinline__ uint4 load8_as_bf16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint4 load8_as_bf16(const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  uint4 r;
  r.x = pack_bf2(a.x, a.y); r.y = pack_bf2(a.z, a.w);
  r.z = pack_bf2(b.x, b.y); r.w = pack_bf2(b.z, b.w);
  return r;
}

// Load 4 consecutive elements as floats.
__device__ __forceinline__ float4 load4f(const uint16_t* p) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  return float4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}
__device__ __forceinline__ float4 load4f(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Store 4 floats as 4 consecutive elements.
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf2(a, b), pack_bf2(c, d)};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
}

__device__ __forceinline__ float ld1(const uint16_t* p) { return bf2f(*p); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }

// GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (Hendrycks &
// Gimpel's approximation), in fp32 with the device library's tanhf.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  return 0.5f * x * (1.0f + tanhf(u));
}

// global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane l
// lands at the wave-uniform LDS address lptr + 16 l.
#define PTDIT_GLDS16(gptr, lptr)                                                                 \
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(gptr),       \
                                   (void __attribute__((address_space(3)))*)(lptr), 16, 0, 0)

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] at [15:14]); n must be a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}

}  // namespace ptdit
