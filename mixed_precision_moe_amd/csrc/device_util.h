// device_util.h -- small gfx950 device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

struct u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t pair) {
  return __uint_as_float(pair << 16);
}
__device__ __forceinline__ float bf16hi_to_f32(uint32_t pair) {
  return __uint_as_float(pair & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return u32x4{v.x, v.y, v.z, v.w};
}

// Non-temporal 16-byte load for data read exactly once (weights).
__device__ __forceinline__ u32x4 load_u32x4_stream(const void* p) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return u32x4{v[0], v[1], v[2], v[3]};
}

// Values the hardware holds once per wave (tile entries, expert handles): read
// them from lane 0 so the compiler keeps them, and whatever is derived from
// them, in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Buffer resource over [base, base + bytes): loads through it take their
// offsets in an SGPR (wave-uniform part) plus one VGPR (per-lane part), and a
// load outside the range returns zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16-byte load through a buffer resource; stream = non-temporal (read once).
template <bool STREAM>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, STREAM ? 2 : 0);
  return u32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// fp16 value j (0..3) of four packed in a uint2, as fp32
__device__ __forceinline__ float half_of(uint2 v, int j) {
  const uint32_t w = j < 2 ? v.x : v.y;
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? (w >> 16) : (w & 0xffffu)));
}

__device__ __forceinline__ uint16_t buffer_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                    uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  v4u t = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8_t, t);
}

// The two constants of the int4 unpack, made opaque so the compiler keeps the
// mask in an SGPR and the magic in a VGPR and can then select one VOP3
// v_and_or_b32 per register (gfx9 VOP3 takes no literal operand).  Only the
// constants come from asm; the and-or that feeds the MFMA is compiler-visible,
// so the hazard recognizer still sees every VGPR write an MFMA reads.
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

struct Int4Consts {
  uint32_t mask, magic;
};
__device__ __forceinline__ Int4Consts int4_consts() {
  return Int4Consts{opaque_sgpr(0x000f000fu), opaque_vgpr(0x43004300u)};
}

// Eight offset-binary int4 codes (nibble value q+8) of one MFMA k-chunk ->
// eight bf16 operands of value 136 + q, exact.  Nibble j of the word holds
// element 2j and nibble j+4 holds element 2j+1, so each output register is one
// shift and one and-or: 0x4300 | u is the bf16 value 128 + u for u < 16.
__device__ __forceinline__ bf16x8_t int4x8_to_bf16_biased(uint32_t w, Int4Consts c) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  v4u t;
  t[0] = (w & c.mask) | c.magic;
  t[1] = ((w >> 4) & c.mask) | c.magic;
  t[2] = ((w >> 8) & c.mask) | c.magic;
  t[3] = ((w >> 12) & c.mask) | c.magic;
  return __builtin_bit_cast(bf16x8_t, t);
}

// Four offset-binary int8 codes (byte value q+128) -> two registers of bf16
// operands of value 128 + q, exact (integers below 256 fit bf16's 8 bits).
__device__ __forceinline__ uint32_t int8x2_to_bf16_biased(uint32_t w, int shift) {
  const float f0 = (float)((w >> shift) & 0xffu);
  const float f1 = (float)((w >> (shift + 8)) & 0xffu);
  return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
}

__device__ __forceinline__ bf16x8_t int8x8_to_bf16_biased(uint32_t w0, uint32_t w1) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  v4u t;
  t[0] = int8x2_to_bf16_biased(w0, 0);
  t[1] = int8x2_to_bf16_biased(w0, 16);
  t[2] = int8x2_to_bf16_biased(w1, 0);
  t[3] = int8x2_to_bf16_biased(w1, 16);
  return __builtin_bit_cast(bf16x8_t, t);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (about 1 ulp
// each; the result is rounded to bf16 afterwards).  Large |g| saturate to the
// right limits: e^-g -> inf gives g * 0, e^-g -> 0 gives g.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * g));
}

}  // namespace moe
