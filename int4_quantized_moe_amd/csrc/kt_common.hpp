// Device helpers shared by the gfx950 kernels of the RAWINT4 routed-expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kt {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 32;  // RAWINT4 group size along K

// ---------------------------------------------------------------- scalar conversions

__device__ __forceinline__ float bf16_to_float(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t float_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// 2^d as fp16 bits for d <= 0 (0 below the smallest subnormal)
__device__ __forceinline__ uint16_t half_pow2_bits(int d) {
  if (d >= -14) return (uint16_t)((d + 15) << 10);
  if (d >= -24) return (uint16_t)(1u << (d + 24));
  return 0;
}

// Exponent p such that maxabs * 2^p < 2^15 (fp16 holds it with headroom);
// 0 for zero or non-finite maxima.
__device__ __forceinline__ int pow2_exponent_for(float maxabs) {
  if (!(maxabs > 0.f) || !(maxabs < INFINITY)) return 0;
  int ex;
  (void)frexpf(maxabs, &ex);  // maxabs = f * 2^ex, f in [0.5, 1)
  return 15 - ex;
}

// Split fp32 v into bf16 hi + lo with v ~= hi + lo (relative error < 2^-16).
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = float_to_bf16(v);
  lo = float_to_bf16(v - bf16_to_float(hi));
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

// 8 fp32 values -> bf16 hi and lo planes (16 bytes each)
__device__ __forceinline__ void split8(const float* v, u32x4& hi, u32x4& lo) {
  uint16_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf16(v[i], h[i], l[i]);
  hi = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
  lo = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
}

// ---------------------------------------------------------------- RAWINT4 decode

// Nonzero scales in [2^-14, 2720] make both decoders exact: (c - 8) * scale is
// an fp16 value, and so are 16 * scale and 24 * scale (24 * 2720 is the largest
// multiple below fp16's maximum that a bf16 scale reaches).
__device__ __forceinline__ bool scale_in_domain(float s) {
  float a = fabsf(s);
  return a == 0.f || (a >= 6.103515625e-05f && a <= 2720.f);
}

// Activation rows in fp16 are stored with every aligned group of 8 elements in
// the order k0 k4 k1 k5 k2 k6 k3 k7, the order in which decode_dword_perm
// produces weights; the position of logical element k:
__host__ __device__ __forceinline__ int perm_pos(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }

// The decoders' nibble masks and fp16 magic values as values the compiler
// cannot see through: with them (w & m) | o becomes one v_and_or_b32 (literal
// operands would make it split the and-or in two).  Made once per kernel.
struct DecodeConsts {
  uint32_t m, o;    // nibble at bits 0-3 of each half; 1024 + c
  uint32_t m6, o6;  // nibble at bits 6-9 of each half; 1 + c / 16
};
__device__ __forceinline__ DecodeConsts decode_consts() {
  uint32_t m = 0x000F000Fu, o = 0x64006400u, m6 = 0x03C003C0u, o6 = 0x3C003C00u;
  asm volatile("" : "+s"(m), "+s"(m6));
  asm volatile("" : "+v"(o), "+v"(o6));
  return DecodeConsts{m, o, m6, o6};
}

// 8 codes of one packed dword, each with one scale s per pair of halves, in the
// order k0 k4 k1 k5 k2 k6 k3 k7, by one fused multiply-add per pair: the code
// sits in the top four mantissa bits of an fp16 1.0 (h = 1 + c / 16), and
// h * 16s - 24s = (c - 8) s.  The product is exact inside the fma, 16s and 24s
// are exact fp16 values for in-domain scales, and so is the result: one
// rounding of an exact value.  s16 = 16 s, b24 = -24 s.
__device__ __forceinline__ u32x4 decode_dword_fma(uint32_t w, half2_t s16, half2_t b24, DecodeConsts dc) {
  auto pair = [&](uint32_t t) {
    const half2_t h = __builtin_bit_cast(half2_t, (t & dc.m6) | dc.o6);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h, s16, b24));
  };
  return u32x4{pair(w << 6), pair(w << 2), pair(w >> 2), pair(w >> 6)};
}

// 8 codes of one packed dword (nibble i = code k_i) -> fp16 weights in the order
// k0 k4 k1 k5 k2 k6 k3 k7.  Pair (k_i, k_{i+4}) is scaled by s[i] (low half for
// k_i, high half for k_{i+4}).  One and-or per pair builds both magic values
// 1024 + c; subtracting 1032 leaves c - 8 exactly.
__device__ __forceinline__ u32x4 decode_dword_perm(uint32_t w, half2_t s0, half2_t s1, half2_t s2, half2_t s3,
                                                   DecodeConsts dc) {
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, (w & dc.m) | dc.o) - bias) * s0);
  r.y = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, ((w >> 4) & dc.m) | dc.o) - bias) * s1);
  r.z = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, ((w >> 8) & dc.m) | dc.o) - bias) * s2);
  r.w = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, ((w >> 12) & dc.m) | dc.o) - bias) * s3);
  return r;
}

// ---------------------------------------------------------------- MXFP4 (E2M1 nibbles)
//
// The MXFP4 weight format (E2M1 codes, a UE8M0 power-of-two scale per group of
// 32, handed over as bf16) is decoded by gfx950's v_cvt_scalef32_pk_f16_fp4:
// one byte (low nibble first) to two fp16 values times 2^(exponent of its fp32
// scale operand), rounded to nearest even.  It reads only the scale's
// exponent, which is all an MXFP4 scale has.

// Nonzero MXFP4 scales must be powers of two in [2^-13, 2^13]: every nonzero
// weight (0.5 .. 6 times the scale) is then a normal fp16 number, exactly.
__device__ __forceinline__ bool scale_in_domain_mxfp4(float s) {
  const uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0) return true;
  return (u & 0x807fffffu) == 0 && s >= 0x1p-13f && s <= 0x1p13f;
}

// The nibbles of one packed dword paired into bytes k_i | k_{i+4} << 4:
// x holds (k0, k4) in byte 0 and (k2, k6) in byte 1, y holds (k1, k5) and (k3, k7).
__device__ __forceinline__ void e2m1_pair_bytes(uint32_t w, uint32_t& x, uint32_t& y) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // bytes k0 k2 k4 k6 | k1 k3 k5 k7
  x = lo | (lo >> 12);
  y = hi | (hi >> 12);
}

__device__ __forceinline__ uint32_t cvt_e2m1(uint32_t v, float s, int sel) {
  half2_t r;
  if (sel == 0)
    r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, s, 0);
  else
    r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, s, 1);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 E2M1 codes of one packed dword, all with the scale s, in the order
// k0 k4 k1 k5 k2 k6 k3 k7 (as decode_dword_fma).
__device__ __forceinline__ u32x4 decode_dword_e2m1(uint32_t w, float s) {
  uint32_t x, y;
  e2m1_pair_bytes(w, x, y);
  return u32x4{cvt_e2m1(x, s, 0), cvt_e2m1(y, s, 0), cvt_e2m1(x, s, 1), cvt_e2m1(y, s, 1)};
}

// 8 E2M1 codes (nibble i = code k_i) in the order k0 k4 k1 k5 k2 k6 k3 k7, pair
// (k_i, k_{i+4}) times the fp16 scales s[i] (as decode_dword_perm): the codes
// are decoded unscaled and multiplied, exact for in-domain scales.
__device__ __forceinline__ u32x4 decode_dword_perm_e2m1(uint32_t w, half2_t s0, half2_t s1, half2_t s2, half2_t s3) {
  uint32_t x, y;
  e2m1_pair_bytes(w, x, y);
  auto mul = [](uint32_t v, half2_t sc) { return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v) * sc); };
  return u32x4{mul(cvt_e2m1(x, 1.f, 0), s0), mul(cvt_e2m1(y, 1.f, 0), s1), mul(cvt_e2m1(x, 1.f, 1), s2),
               mul(cvt_e2m1(y, 1.f, 1), s3)};
}

// 8 fp32 -> bf16 hi (top 16 bits) and lo (top 16 bits of the exact remainder)
__device__ __forceinline__ void split8_trunc(const float* v, u32x4& hi, u32x4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t u = __float_as_uint(v[i]);
    h[i] = u & 0xffff0000u;
    l[i] = __float_as_uint(v[i] - __uint_as_float(h[i]));
  }
  hi = u32x4{(h[0] >> 16) | h[1], (h[2] >> 16) | h[3], (h[4] >> 16) | h[5], (h[6] >> 16) | h[7]};
  lo = u32x4{(l[0] >> 16) | (l[1] & 0xffff0000u), (l[2] >> 16) | (l[3] & 0xffff0000u),
             (l[4] >> 16) | (l[5] & 0xffff0000u), (l[6] >> 16) | (l[7] & 0xffff0000u)};
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ floatx4 mfma_f16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                0, 0);
}

__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 16x16x16 bf16: lane l holds row (A) or column (B) l % 16, contraction values 4 (l / 16) .. + 3
__device__ __forceinline__ floatx4 mfma_bf16_k16(u32x2 a, u32x2 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b), c,
                                                   0, 0, 0);
}

// 4 fp32 -> bf16 hi (top 16 bits) and lo (top 16 bits of the exact remainder)
__device__ __forceinline__ void split4_trunc(float4 v, u32x2& hi, u32x2& lo) {
  const float x[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = __float_as_uint(x[i]) & 0xffff0000u;
    l[i] = __float_as_uint(x[i] - __uint_as_float(h[i]));
  }
  hi = u32x2{(h[0] >> 16) | h[1], (h[2] >> 16) | h[3]};
  lo = u32x2{(l[0] >> 16) | (l[1] & 0xffff0000u), (l[2] >> 16) | (l[3] & 0xffff0000u)};
}

// ---------------------------------------------------------------- 16-lane reductions (DPP)

// The 16 lanes of each DPP row (lanes 16r .. 16r + 15) end with the same result:
// swap neighbours, swap pairs, mirror within 8, mirror within 16.  Every lane
// combines the same operands in a commutative order, so the results are equal
// bit for bit.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f<0xB1>(v);
  v = v + dpp_f<0x4E>(v);
  v = v + dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// ---------------------------------------------------------------- activation

// Sigmoid from the hardware exp2 and reciprocal (about 1 ulp each), with the
// exponent argument clamped so that exp never overflows.
__device__ __forceinline__ float sigmoid_f(float z) {
  const float e = __builtin_amdgcn_exp2f(fminf(-z, 88.f) * 1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.f + e);
}

// ---------------------------------------------------------------- global -> LDS copies

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// 16 bytes from global memory to LDS: lane l's bytes land at lds_base + 16 * l
// (lds_base wave-uniform, through M0).  Counted by vmcnt like any vector load.
// Issued from asm so that the compiler, which cannot tell which ring slot a
// later LDS read touches, does not drain every outstanding copy before it; the
// ring's explicit vmcnt waits order the copies and the reads instead.  M0 is
// declared clobbered, so the compiler keeps no value of its own in it across
// a copy (it treats M0 as reserved and warns about naming it; the warning is
// for a save and restore the kernels do not need).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  // one wait state between the M0 write and the load that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(base)
               : "memory", "m0");
}

// 4 bytes from global memory to LDS: lane l's bytes land at lds_base + 4 * l.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt in 6:4 left at its maximum, lgkmcnt in 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

}  // namespace kt
