// Device-side definitions shared by the MX quantiser and the fused attention
// kernel (gfx950 / CDNA4).
//
// Element formats are those of the OCP Microscaling Formats v1.0
// specification, which the pages name as MXFP8, MXFP6 and MXFP4
// (Fused-Softmax for efficient quantized attention, summary).
//
// Matrix-core facts used here (scaled MFMA V_MFMA_SCALE_F32_16X16X128_F8F6F4,
// measured on gfx950 with one-hot probes):
//   * A is 16 x 128 (rows x K), B is 128 x 16 (K x columns), C is 16 x 16;
//     lane l = 16*g + r holds row r of A / column r of B, and C rows 4g..4g+3
//     of column r.
//   * FP6 and FP4 operands: lane (g, r) holds the 32 consecutive K elements
//     [32g, 32g+32) (a little-endian bit stream, element i at bit bits*i) and
//     its scale byte applies to exactly those: one lane = one MX block.
//   * FP8 operands: lane (g, r) holds K elements [16g, 16g+16) in bytes 0-15
//     and [64+16g, 64+16g+16) in bytes 16-31; the scale for K block c
//     (elements [32c, 32c+32)) is the scale operand of lane group c.
//   * The scaled conversions divide by their scale operand, round to nearest
//     even; FP4/FP6 saturate, FP8 overflows to NaN.  The FP6 32-element
//     conversion places element i of its first source at bit 12i and element
//     i of its second source at bit 12i+6.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));

enum { FMT_E4M3 = 0, FMT_E2M3 = 1, FMT_E2M1 = 2 };
// FP6 E3M2: a probability format only (P~ over E2M3 operands), never an
// operand format of a launch, so it has no bit in a format set.
enum { FMT_E3M2 = 3 };

// Per-format constants.  emax: exponent of the largest normal binade;
// e_top: its biased exponent; cap: the largest upward block shift that keeps
// the E8M0 byte 127 - emax - shift >= 0.
template <int F> struct Fmt;
template <> struct Fmt<FMT_E4M3> {
  static constexpr int bits = 8, mbits = 3, bias = 7, emax = 8, e_top = 15;
  static constexpr int mfma = 0;                 // cbsz / blgp operand format code
  static constexpr float maxval = 448.0f;
  static constexpr uint32_t one_code = 0x38;     // 1.0
};
template <> struct Fmt<FMT_E2M3> {
  static constexpr int bits = 6, mbits = 3, bias = 1, emax = 2, e_top = 3;
  static constexpr int mfma = 2;
  static constexpr float maxval = 7.5f;
  static constexpr uint32_t one_code = 0x08;
};
template <> struct Fmt<FMT_E2M1> {
  static constexpr int bits = 4, mbits = 1, bias = 1, emax = 2, e_top = 3;
  static constexpr int mfma = 4;
  static constexpr float maxval = 6.0f;
  static constexpr uint32_t one_code = 0x2;
};
template <> struct Fmt<FMT_E3M2> {
  static constexpr int bits = 6, mbits = 2, bias = 3, emax = 4, e_top = 7;
  static constexpr int mfma = 3;
  static constexpr float maxval = 28.0f;
  static constexpr uint32_t one_code = 0x0C;
};

// Calls fn(std::integral_constant<int, F>) for the element format f, which
// must be in the bit set FSET (1 << FMT_*); with a single format the call
// is direct and f is not read.
template <int FSET, typename Fn>
__device__ __forceinline__ void with_format(int f, Fn&& fn) {
  if constexpr (FSET == (1 << FMT_E4M3)) fn(std::integral_constant<int, FMT_E4M3>{});
  else if constexpr (FSET == (1 << FMT_E2M3)) fn(std::integral_constant<int, FMT_E2M3>{});
  else if constexpr (FSET == (1 << FMT_E2M1)) fn(std::integral_constant<int, FMT_E2M1>{});
  else {
    if constexpr ((FSET >> FMT_E4M3) & 1) {
      if (f == FMT_E4M3) { fn(std::integral_constant<int, FMT_E4M3>{}); return; }
    }
    if constexpr ((FSET >> FMT_E2M3) & 1) {
      if (f == FMT_E2M3) { fn(std::integral_constant<int, FMT_E2M3>{}); return; }
    }
    if constexpr ((FSET >> FMT_E2M1) & 1) {
      if (f == FMT_E2M1) { fn(std::integral_constant<int, FMT_E2M1>{}); return; }
    }
  }
}

// Matrix-core operand of 32 elements in the format's packing: FP8 8 dwords,
// FP6 6 dwords, FP4 4 dwords.  The narrow FP6/FP4 vectors keep registers
// free that 8-dword operands would fill with zeros.
template <int F> struct Operand;
template <> struct Operand<FMT_E4M3> { typedef v8i type; static constexpr int words = 8; };
template <> struct Operand<FMT_E2M3> { typedef v6i type; static constexpr int words = 6; };
template <> struct Operand<FMT_E2M1> { typedef v4i type; static constexpr int words = 4; };
template <> struct Operand<FMT_E3M2> { typedef v6i type; static constexpr int words = 6; };
template <int F> using opv = typename Operand<F>::type;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// floor(log2(a)) of a finite a > 0 (fp32 subnormals included).
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF);
  if (e != 0) return e - 127;
  return (31 - __clz(u & 0x7FFFFF)) - 149;
}

// Convert 32 fp32 values to packed element codes: each value is divided by
// a power-of-two scale (exact) and rounded to nearest even, saturating.
// Elements 0-15 use s_lo and 16-31 use s_hi (one FP8 lane holds two half
// blocks); FP6/FP4 lanes hold one block and use s_lo for all 32.  Output
// words follow the operand packing: FP8 8 words, FP6 6 words, FP4 4 words.
// FP8 saturation needs an explicit clamp (the conversion overflows to NaN);
// callers whose scaled values provably stay in range pass CLAMP = false.
template <int F, bool CLAMP> struct Pack32;

template <bool CLAMP> struct Pack32<FMT_E4M3, CLAMP> {
  static __device__ __forceinline__ float sat(float v) {
    return CLAMP ? __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f) : v;
  }
  static __device__ __forceinline__ void run(const float* y, uint32_t* w, float s_lo = 1.0f,
                                             float s_hi = 1.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sc = i < 4 ? s_lo : s_hi;
      // each conversion writes one 16-bit half and keeps the other; the
      // starting value is overwritten in full, so any register will do (one
      // whose value dies here costs no copy)
      v2s lo = __builtin_bit_cast(v2s, y[4 * i + 1]);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, sat(y[4 * i + 0]), sat(y[4 * i + 1]), sc, false);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, sat(y[4 * i + 2]), sat(y[4 * i + 3]), sc, true);
      w[i] = __builtin_bit_cast(uint32_t, lo);
    }
  }
};

// The 32-element FP6 conversion reads 32 source VGPRs over several cycles.
// Issued through the builtin, the compiler may give it a destination that
// overlaps its sources and rewrite those sources on the next instruction,
// which corrupts the result.  Issue it with an early-clobber destination and
// wait states before anything can overwrite its sources.
template <bool CLAMP> struct Pack32<FMT_E2M3, CLAMP> {
  static __device__ __forceinline__ void run(const float* y, uint32_t* w, float s_lo = 1.0f,
                                             float = 1.0f) {
    v16f ev, od;
#pragma unroll
    for (int i = 0; i < 16; ++i) { ev[i] = y[2 * i]; od[i] = y[2 * i + 1]; }
    v6i r;
    asm volatile(
        "v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3\n\t"
        "s_nop 7\n\t"
        "s_nop 7"
        : "=&v"(r)
        : "v"(ev), "v"(od), "v"(s_lo));
#pragma unroll
    for (int i = 0; i < 6; ++i) w[i] = (uint32_t)r[i];
  }
};

// FP6 pack of 32 values held as even elements (v[0..15]) then odd elements
// (v[16..31]): the two sources of the 32-element conversion, so that callers
// can produce them in place.  Same conversion and wait states as above;
// F = FMT_E3M2 takes the E3M2 ("bf6") form of the conversion.
template <int F = FMT_E2M3>
__device__ __forceinline__ void pack_fp6_split(const float* v, uint32_t* w, float scale) {
  static_assert(F == FMT_E2M3 || F == FMT_E3M2, "FP6 formats");
  v16f ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) { ev[i] = v[i]; od[i] = v[16 + i]; }
  v6i r;
  if constexpr (F == FMT_E2M3)
    asm volatile(
        "v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3\n\t"
        "s_nop 7\n\t"
        "s_nop 7"
        : "=&v"(r)
        : "v"(ev), "v"(od), "v"(scale));
  else
    asm volatile(
        "v_cvt_scalef32_2xpk16_bf6_f32 %0, %1, %2, %3\n\t"
        "s_nop 7\n\t"
        "s_nop 7"
        : "=&v"(r)
        : "v"(ev), "v"(od), "v"(scale));
#pragma unroll
  for (int i = 0; i < 6; ++i) w[i] = (uint32_t)r[i];
}

template <bool CLAMP> struct Pack32<FMT_E2M1, CLAMP> {
  static __device__ __forceinline__ void run(const float* y, uint32_t* w, float s_lo = 1.0f,
                                             float = 1.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the four conversions write the four bytes of r, so its starting
      // value does not matter (one that dies here costs no move)
      uint32_t r = __float_as_uint(y[8 * i + 1]);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * i + 0], y[8 * i + 1], s_lo, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * i + 2], y[8 * i + 3], s_lo, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * i + 4], y[8 * i + 5], s_lo, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * i + 6], y[8 * i + 7], s_lo, 3);
      w[i] = r;
    }
  }
};

}  // namespace fsa
