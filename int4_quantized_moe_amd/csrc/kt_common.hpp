// Device helpers shared by the gfx950 kernels of the RAWINT4 routed-expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kt {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
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

// Nonzero scales in [2^-14, 8160] make (c - 8) * scale exact in fp16.
__device__ __forceinline__ bool scale_in_domain(float s) {
  float a = fabsf(s);
  return a == 0.f || (a >= 6.103515625e-05f && a <= 8160.f);
}

// fp16 pair ((c0 - 8) * s0, (c1 - 8) * s1) from nibble codes c0, c1 in [0, 15].
// 0x6400 | c is the fp16 value 1024 + c; subtracting 1032 leaves c - 8 exactly,
// and the product with an in-domain scale is exact.
__device__ __forceinline__ uint32_t decode_pair(uint32_t c0, uint32_t c1, half2_t s) {
  uint32_t magic = c0 | (c1 << 16) | 0x64006400u;
  half2_t v = __builtin_bit_cast(half2_t, magic);
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  v = (v - bias) * s;
  return __builtin_bit_cast(uint32_t, v);
}

// Activation rows in fp16 are stored with every aligned group of 8 elements in
// the order k0 k4 k1 k5 k2 k6 k3 k7, the order in which decode_dword_perm
// produces weights; the position of logical element k:
__host__ __device__ __forceinline__ int perm_pos(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }

// The decode's nibble mask and fp16 magic as values the compiler cannot see
// through: with them (w & m) | o becomes one v_and_or_b32 (literal operands
// would make it split the and-or in two).  Made once per kernel.
struct DecodeConsts {
  uint32_t m, o;
};
__device__ __forceinline__ DecodeConsts decode_consts() {
  uint32_t m = 0x000F000Fu, o = 0x64006400u;
  asm volatile("" : "+s"(m));
  asm volatile("" : "+v"(o));
  return DecodeConsts{m, o};
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

// 8 consecutive codes of one packed dword (low nibble first) -> 8 fp16 values
// in natural k order, all with scale s.
__device__ __forceinline__ u32x4 decode_dword(uint32_t w, half2_t s) {
  u32x4 r;
  r.x = decode_pair(w & 15u, (w >> 4) & 15u, s);
  r.y = decode_pair((w >> 8) & 15u, (w >> 12) & 15u, s);
  r.z = decode_pair((w >> 16) & 15u, (w >> 20) & 15u, s);
  r.w = decode_pair((w >> 24) & 15u, w >> 28, s);
  return r;
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
// not used by anything else in these kernels.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  // one wait state between the M0 write and the load that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(base) : "memory");
}

// 4 bytes from global memory to LDS: lane l's bytes land at lds_base + 4 * l.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(base) : "memory");
}

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt in 6:4 left at its maximum, lgkmcnt in 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

}  // namespace kt
