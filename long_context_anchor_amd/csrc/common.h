// Device helpers shared by the gfx950 kernels of libkascade.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define KC_INLINE __device__ __forceinline__

namespace kc {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 2^x on the hardware exp unit (v_exp_f32).  Arguments are <= 0 wherever the
// kernels call it, and results that underflow flush to 0.
KC_INLINE float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
KC_INLINE float log2f_fast(float x) { return __builtin_amdgcn_logf(x); }

// bf16 <-> fp32.  bf16 is the high half of an fp32 word.
KC_INLINE float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
KC_INLINE float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// fp32 -> bf16, round to nearest even, on the hardware converter
// (v_cvt_pk_bf16_f32).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
KC_INLINE uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
KC_INLINE uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// dot of two bf16 pairs accumulated in fp32 (v_dot2c_f32_bf16).
KC_INLINE float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// fp16 counterparts (IEEE half): v_dot2c_f32_f16 and round-to-nearest-even
// packing on the hardware converter.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
KC_INLINE float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}
KC_INLINE uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
}
KC_INLINE float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w).x;
}

// 16-bit element formats of the bf16/fp16 kernels.
template <bool HALF>
struct Fmt16;
template <>
struct Fmt16<false> {   // bf16
  typedef bf16x8_t v8;
  static KC_INLINE float dot2(uint32_t a, uint32_t b, float c) { return dot2_bf16(a, b, c); }
  static KC_INLINE uint32_t pack(float lo, float hi) { return pack_bf16x2(lo, hi); }
  static KC_INLINE f32x16_t mfma(const v8& a, const v8& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Fmt16<true> {    // fp16
  typedef f16x8_t v8;
  static KC_INLINE float dot2(uint32_t a, uint32_t b, float c) { return dot2_f16(a, b, c); }
  static KC_INLINE uint32_t pack(float lo, float hi) { return pack_f16x2(lo, hi); }
  static KC_INLINE f32x16_t mfma(const v8& a, const v8& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Cross-lane moves inside a 16-lane DPP row (GFX9 DPP controls).
enum : int {
  DPP_XOR1 = 0xB1,          // quad_perm [1,0,3,2]
  DPP_XOR2 = 0x4E,          // quad_perm [2,3,0,1]
  DPP_HALF_MIRROR = 0x141,  // lane i <- i ^ 7 within 8 lanes
  DPP_MIRROR = 0x140,       // lane i <- i ^ 15 within 16 lanes
};
template <int CTRL>
KC_INLINE float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row; every lane receives the total.
KC_INLINE float row16_sum(float x) {
  x += dpp_f<DPP_MIRROR>(x);
  x += dpp_f<DPP_HALF_MIRROR>(x);
  x += dpp_f<DPP_XOR2>(x);
  x += dpp_f<DPP_XOR1>(x);
  return x;
}
KC_INLINE float row16_max(float x) {
  x = fmaxf(x, dpp_f<DPP_MIRROR>(x));
  x = fmaxf(x, dpp_f<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f<DPP_XOR2>(x));
  x = fmaxf(x, dpp_f<DPP_XOR1>(x));
  return x;
}

KC_INLINE float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
KC_INLINE float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Order-preserving map from fp32 to uint32 (larger float -> larger key).
// -0.0 is folded onto +0.0 first.
KC_INLINE uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-byte global load / store.
KC_INLINE uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
KC_INLINE uint4 ld16_nt(const void* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace kc
