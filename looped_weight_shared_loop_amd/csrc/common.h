// Device helpers shared by the gfx950 kernels of the looped decoder.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

DEV float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round to nearest, ties to even: one v_cvt_pk_bf16_f32.
DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// Two floats to a packed bf16 pair (a in the low half).
DEV uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

DEV float round_to(float v, bf16_t*) { return bf2f(f2bf(v)); }
DEV float round_to(float v, float*) { return v; }

// Element I/O for the two storage types.
DEV float ld1(const float* p) { return *p; }
DEV float ld1(const bf16_t* p) { return bf2f(*p); }
DEV void st1(float* p, float v) { *p = v; }
DEV void st1(bf16_t* p, float v) { *p = f2bf(v); }

// 8 consecutive elements (16 B for bf16, 32 B for fp32); p must be aligned.
DEV void ld8(const bf16_t* p, float* v) {
  uint4 q = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
DEV void ld8(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
DEV void st8(bf16_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
DEV void st8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// v combined with v of lane l ^ 32 (l ^ 16) without an LDS round trip:
// v_permlane32_swap (v_permlane16_swap) exchanges the odd 32- (16-) lane rows
// of one copy of v with the even rows of another, so each lane ends up with
// its own value in one copy and its partner's in the other.  Sum and max are
// commutative, so the results equal those of a shuffle bit for bit.
DEV void xswap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
DEV void xswap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
DEV float x32_sum(float v) { float a, b; xswap32(v, a, b); return a + b; }
DEV float x32_max(float v) { float a, b; xswap32(v, a, b); return fmaxf(a, b); }
DEV float x16_sum(float v) { float a, b; xswap16(v, a, b); return a + b; }
DEV float x16_max(float v) { float a, b; xswap16(v, a, b); return fmaxf(a, b); }

DEV float wave_sum(float v) {
  v = x16_sum(x32_sum(v));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEV float wave_max(float v) {
  v = x16_max(x32_max(v));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

DEV bf16x8_t as_bf16x8(uint4 q) { return __builtin_bit_cast(bf16x8_t, q); }
DEV bf16x8_t as_bf16x8(u32x4_t q) { return __builtin_bit_cast(bf16x8_t, q); }
DEV u32x4_t ldv4(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
DEV void stv4(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

DEV f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
DEV f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware instruction alone (about 1 ulp; results below
// 2^-126 flush to zero): the softmax exponentials, where such tiny
// probabilities do not matter, skip the denormal-range handling of exp2f.
DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// x sigma(x) = x / (1 + e^-x) from the hardware 2^x and reciprocal (about
// 1 ulp each): a few instructions instead of a library exponential and an
// IEEE division.  Large negative x give 1 / inf = 0, so the result is 0.
DEV float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-1.4426950408889634f * x)); }

