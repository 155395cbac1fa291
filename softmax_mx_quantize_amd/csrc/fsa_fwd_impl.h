// Fused-Softmax attention forward on gfx950 scaled MFMA (MXFP8/6/4): the
// kernel templates, included by one translation unit per build flavour
// (fsa_fwd.hip for E2M3/E2M1, fsa_fwd_e4m3.hip for E4M3).
//
// What is computed (Fused-Softmax for efficient quantized attention, summary;
// Moving softmax to matrix operations speeds up AI inference by over 2x,
// "Read it as" and the "How it works" figure), with the readings fixed in the
// oracle's module documentation:
//   1. frozen max per query row from the first 128 keys, in binades:
//      max(window max, mean + (sqrt(2 ln n) + 1) * std) + bias;
//   2. scores on the matrix cores with the exponential's linear part folded
//      in: Q carries log2(e)/sqrt(D) (applied when it is quantised), 2^23
//      rides on Q's E8M0 scale, and the accumulator starts at
//      2^23 (127 + R) - 2^23 m~, so each fp32 output y already is the
//      exponent-field value of the bit-pattern exponential;
//   3. epilogue per 32-key MX block: one truncating conversion per element
//      turns y into the fp32 pattern of 2^(t + R); the block's binade comes
//      from the largest pattern, and the scaled pack conversion divides by the
//      block's power-of-two shift and rounds onto the element grid: the
//      exponential and the MX quantisation of P with no exp instruction;
//   4. O^T += V^T P~^T and l += 1 P~^T on the matrix cores (same P~ in
//      numerator and denominator, as EFQ-Softmax: Exp-Free Quantization for
//      Softmax, abstract, uses it);
//   5. a block above the guess takes a larger E8M0 scale, which is the
//      whole-binade re-basing of the fallback up to a common power of two;
//      rows beyond 64 binades are recomputed by the fallback kernel;
//   6. out = bf16(O / l).
//
// Work decomposition.  One workgroup = NWAVES waves = NWAVES*16*NSUB query
// rows of one (batch, head).  Key tiles of 128 keys (K^ rows and the matching
// V^T columns, with their E8M0 scales) stream through an LDS ring filled by
// direct global->LDS buffer loads.  Each wave keeps its queries' Q^
// fragments, O^T accumulators and row sums in registers; there is no online
// max and no rescaling.  Two waves share each SIMD (two workgroups of four
// waves per CU by default), and the hardware overlaps one wave's vector
// epilogue with the other's MFMAs.
//
// Register layout (16x16x128 scaled MFMA).  Lane (g, r) = 16g + r.  The score
// tile is computed transposed (keys as rows, queries as columns) so that a
// lane ends up with 32 keys of one query: the K^ rows are gathered from LDS
// in the order that makes those 32 keys exactly the keys this lane must
// supply as the B operand of the P V product.  For FP6/FP4 that is one whole
// MX block of P; for FP8 it is two half blocks, completed with the lane
// 16 apart.
//
// LDS layout.  Every K^ row and V^T row occupies 128 bytes (8 chunks of 16
// bytes; FP6/FP4 rows leave chunks unused).  Chunk c of row R is stored at
// chunk c ^ f(R): the XOR swizzle makes the 8 lanes that read the same
// logical chunk of 8 different rows hit 8 different bank groups.  Scale bytes
// arrive tile-ordered (see the quantiser's layouts), one 8-byte read per
// lane per tile and operand.
#pragma once

#include <type_traits>

#include "fsa_device.h"
#include "fsa_internal.h"
#include "lds_dma.h"

// Build-time knobs (the defaults are the measured best): waves per SIMD the
// kernels are built for, fragment pipeline depth (-1: per format), query
// subtiles per wave and waves per workgroup for each element format.
#ifndef FSA_WPE
#define FSA_WPE 2
#endif
#ifndef FSA_PIPE
#define FSA_PIPE -1
#endif
#ifndef FSA_NSUB6
#define FSA_NSUB6 2
#endif
#ifndef FSA_NSUB4
#define FSA_NSUB4 2
#endif
#ifndef FSA_NSUB8
#define FSA_NSUB8 2
#endif
#ifndef FSA_NW8
#define FSA_NW8 4
#endif
#ifndef FSA_NW6
#define FSA_NW6 4
#endif
#ifndef FSA_NW4
#define FSA_NW4 4
#endif

namespace fsa {

// The builtin of the scaled MFMA only takes 8-dword operands; the narrow
// FP6/FP4 forms of the same intrinsic are reached through its overloaded
// LLVM name.  (Compiler instructions: the hazard handling is the same.)
__device__ v4f mfma_scale_v6(v6i a, v6i b, v4f c, int cbsz, int blgp, int opsel_a, int sa,
                             int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v6i32.v6i32");
__device__ v4f mfma_scale_v4(v4i a, v4i b, v4f c, int cbsz, int blgp, int opsel_a, int sa,
                             int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v4i32");
// Mixed widths: an FP4 A operand with an FP8 or FP6 B operand.
__device__ v4f mfma_scale_v4_v8(v4i a, v8i b, v4f c, int cbsz, int blgp, int opsel_a, int sa,
                                int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v8i32");
__device__ v4f mfma_scale_v4_v6(v4i a, v6i b, v4f c, int cbsz, int blgp, int opsel_a, int sa,
                                int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v6i32");

namespace {

constexpr int KT = 128;          // keys per tile
constexpr float MAGIC = 12582912.0f;   // 1.5 * 2^23: float + MAGIC rounds to an integer
// A score equal to the reference gives the fp32 pattern of 2^REF, so scores
// from 188 binades below it to 66 above map to normal fp32 numbers.
constexpr int REF = 62;

// Binade of a block relative to the reference, in element codes:
// floor(RNE(2^M (y / 2^23 - 127 - REF)) / 2^M) for the block's largest
// exponent-field value y.  y * 2^(M-23) is exact, and adding the integer
// constant plus MAGIC rounds once, to nearest even.  Blocks whose largest
// value lies below 2^-(127+REF) (or that are fully masked, y = -inf) count as
// y = 0, which already puts them beyond the largest block shift.  Values
// more than HI_BINADE binades above the reference count as exactly that
// many (the MAGIC window holds 2^22 codes); the row then falls back with
// kappa = HI_BINADE, which is exact for every score within 2^18 binades of
// its frozen max.
constexpr int HI_BINADE = 1 << 18;
// Largest guess-relative block binade the main sweep absorbs by block shifts
// alone; rows above it go to the fallback kernel.
constexpr int EXT = 64;
static_assert(HI_BINADE > EXT, "clamped binades must reach the fallback kernel");
template <int M>
__device__ __forceinline__ int block_binade(float y) {
  const float yc = __builtin_amdgcn_fmed3f(y, 0.0f, 8388608.0f * (float)(127 + REF + HI_BINADE));
  const float t = __builtin_fmaf(yc, (float)(1 << M) * 0x1p-23f,
                                 MAGIC - (float)((1 << M) * (127 + REF)));
  return (int)(__float_as_uint(t) - __float_as_uint(MAGIC)) >> M;
}

// Divisor of the scaled conversions for a block whose P~ scale byte is sb:
// 2^(sb + REF - 127), taking the bit-pattern value 2^(t + REF) to
// 2^(t + pl + Delta).
__device__ __forceinline__ float conv_scale(int sb) {
  return __uint_as_float((uint32_t)(sb + REF) << 23);
}

// Level of a block whose largest pattern is m: the binade plus 127 + REF,
// i.e. the exponent field of m after rounding its mantissa to M bits
// (nearest, ties to even): floor(RNE(2^M m / 2^23) / 2^M).  For a pattern
// from y >= 2^23 this is the binade of block_binade below; smaller patterns
// lie below every level the shifts distinguish.  m is clamped first so that
// the rounding cannot carry out of 32 bits; the clamp sits one level above
// the largest shift (127 + REF + EXT), so the row still reaches the
// fallback.
template <int M>
__device__ __forceinline__ int block_level(uint32_t m) {
  constexpr uint32_t LIM = (uint32_t)(127 + REF + EXT + 1) << 23;
  const uint32_t mc = min(m, LIM);
  const uint32_t lsb = (mc >> (23 - M)) & 1u;
  return (int)((mc + (1u << (22 - M)) - 1u + lsb) >> 23);
}

typedef __attribute__((address_space(3))) void lds_void;


// Truncation toward zero to u32 (v_cvt_u32_f32, which saturates and maps NaN
// and negatives to 0; the exponential relies on that).  It must stay a
// compiler-visible conversion: the epilogue feeds it straight from MFMA
// results, and only instructions the compiler sees get the wait states that
// reading an MFMA result requires.  Its input must come straight from the
// product (never a select with constants), so that no out-of-range case can
// be folded away at compile time; masking happens on the integer result.
__device__ __forceinline__ uint32_t cvt_u32_trunc(float y) {
  return (uint32_t)y;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

// Position p (0..31) of a lane's operand list -> index along the 128-wide K
// dimension for lane group g.
template <int F>
__device__ __forceinline__ int kpos(int g, int p) {
  if (Fmt<F>::bits == 8) return p < 16 ? 16 * g + p : 64 + 16 * g + (p - 16);
  return 32 * g + p;
}

// XOR swizzles (16-byte chunk index within a 128-byte LDS row), so that
// the lanes the LDS serves together read distinct banks (64 banks of 4
// bytes: two rows per bank line, the row's parity picks the half).  FP8 and
// FP4 fragments are 16-byte reads, served 8 lanes at a time: the 8 rows of
// lanes r = 0..7 need distinct chunks within each parity.  FP6 fragments
// are three 8-byte reads, served 16 or more lanes at a time: all 16 rows of
// a lane group need distinct 8-byte slots, i.e. distinct chunks within each
// parity over 8 rows (a lane's score-product rows are 32 (r/4) + r%4 + 4j,
// its output-product rows r + 16 dt).
template <int F, int D>
__device__ __forceinline__ int swz_k(int row) {
  if (D != 128) return 0;
  if (Fmt<F>::bits == 6) return ((row >> 1) & 1) | (((row >> 5) & 3) << 1);
  const int hi = Fmt<F>::bits == 8 ? (row >> 4) & 1 : (row >> 5) & 1;
  return (row & 3) | (hi << 2);
}
template <int F>
__device__ __forceinline__ int swz_v(int row) { return Fmt<F>::bits == 6 ? (row >> 1) & 7 : row & 7; }

// A lane's 32 operand elements along a 128-byte swizzled LDS row.  `len` is
// the number of valid K elements of the row (elements past it are zero).
template <int F>
__device__ __forceinline__ opv<F> lds_operand(const uint8_t* row, int sw, int g, int len) {
  opv<F> o = zero_operand<F>();
  if constexpr (Fmt<F>::bits == 8) {
    if (16 * g < len) {
      uint4 a = *reinterpret_cast<const uint4*>(row + 16 * (g ^ sw));
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    }
    if (64 + 16 * g < len) {
      uint4 b = *reinterpret_cast<const uint4*>(row + 16 * ((4 + g) ^ sw));
      o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
  } else if constexpr (Fmt<F>::bits == 6) {
    if (32 * g < len) {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int off = 24 * g + 8 * i;
        uint2 a = *reinterpret_cast<const uint2*>(row + 16 * ((off >> 4) ^ sw) + (off & 15));
        o[2 * i] = a.x; o[2 * i + 1] = a.y;
      }
    }
  } else {
    if (32 * g < len) {
      uint4 a = *reinterpret_cast<const uint4*>(row + 16 * (g ^ sw));
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    }
  }
  return o;
}

// The same 32 elements straight from global memory (unswizzled row).
template <int F>
__device__ __forceinline__ opv<F> global_operand(const uint8_t* row, int g, int len) {
  opv<F> o = zero_operand<F>();
  if constexpr (Fmt<F>::bits == 8) {
    if (16 * g < len) {
      uint4 a = *reinterpret_cast<const uint4*>(row + 16 * g);
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    }
    if (64 + 16 * g < len) {
      uint4 b = *reinterpret_cast<const uint4*>(row + 64 + 16 * g);
      o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
  } else if constexpr (Fmt<F>::bits == 6) {
    if (32 * g < len) {
      const uint2* p = reinterpret_cast<const uint2*>(row + 24 * g);
      uint2 a = p[0], b = p[1], c = p[2];
      o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y; o[4] = c.x; o[5] = c.y;
    }
  } else {
    if (32 * g < len) {
      uint4 a = *reinterpret_cast<const uint4*>(row + 16 * g);
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    }
  }
  return o;
}

// The scaled MFMA with operands of the format's own width (declared above,
// outside this namespace).

// OA selects the byte of `sa` that scales A (op_sel); B's scale is byte 0.
template <int F, int OA = 0>
__device__ __forceinline__ v4f mfma(const opv<F>& a, const opv<F>& b, const v4f& c, int sa, int sb) {
  if constexpr (Fmt<F>::bits == 8)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma,
                                                            OA, sa, 0, sb);
  else if constexpr (Fmt<F>::bits == 6)
    return mfma_scale_v6(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma, OA, sa, 0, sb);
  else
    return mfma_scale_v4(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma, OA, sa, 0, sb);
}
// The same with A's scale byte chosen by a value that is a constant after
// unrolling.
template <int F>
__device__ __forceinline__ v4f mfma_sel(const opv<F>& a, const opv<F>& b, const v4f& c, int sa,
                                        int byte, int sb) {
  switch (byte & 3) {
    case 0: return mfma<F, 0>(a, b, c, sa, sb);
    case 1: return mfma<F, 1>(a, b, c, sa, sb);
    case 2: return mfma<F, 2>(a, b, c, sa, sb);
    default: return mfma<F, 3>(a, b, c, sa, sb);
  }
}

// Row sums l += 1 P~^T on the matrix core: the all-ones A operand is held
// in FP4 (E2M1 1.0 = 0x2 in every nibble, 4 registers) whatever the format
// of P~; FP4 ones times P~ in its own format is the same exact sum.
__device__ __forceinline__ v4i ones_fp4() {
  v4i o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = 0x22222222;
  return o;
}
template <int F>
__device__ __forceinline__ v4f row_sum(const v4i& ones, const opv<F>& p, const v4f& c, int sp) {
  if constexpr (Fmt<F>::bits == 8)
    return mfma_scale_v4_v8(ones, p, c, Fmt<FMT_E2M1>::mfma, Fmt<F>::mfma, 0, 127, 0, sp);
  else if constexpr (Fmt<F>::bits == 6)
    return mfma_scale_v4_v6(ones, p, c, Fmt<FMT_E2M1>::mfma, Fmt<F>::mfma, 0, 127, 0, sp);
  else
    return mfma_scale_v4(ones, p, c, Fmt<FMT_E2M1>::mfma, Fmt<F>::mfma, 0, 127, 0, sp);
}

template <int F>
__device__ __forceinline__ opv<F> ones_operand() {
  constexpr int BITS = Fmt<F>::bits;
  constexpr uint32_t c = Fmt<F>::one_code;
  opv<F> o = zero_operand<F>();
  if constexpr (BITS == 8) {
    for (int i = 0; i < 8; ++i) o[i] = (int)(c * 0x01010101u);
  } else if constexpr (BITS == 4) {
    for (int i = 0; i < 4; ++i) o[i] = (int)(c * 0x11111111u);
  } else {
    // 32 six-bit fields: 4 fields make 3 bytes, repeated.
    const uint32_t w24 = c | (c << 6) | (c << 12) | (c << 18);
    const uint8_t b0 = w24 & 0xFF, b1 = (w24 >> 8) & 0xFF, b2 = (w24 >> 16) & 0xFF;
    uint8_t bytes[24];
    for (int i = 0; i < 8; ++i) { bytes[3 * i] = b0; bytes[3 * i + 1] = b1; bytes[3 * i + 2] = b2; }
    for (int i = 0; i < 6; ++i)
      o[i] = (int)(bytes[4 * i] | (bytes[4 * i + 1] << 8) | (bytes[4 * i + 2] << 16) |
                   ((uint32_t)bytes[4 * i + 3] << 24));
  }
  return o;
}

// Cross-lane exchanges on the vector unit (v_permlane16/32_swap; the swap
// trades the odd 16-lane rows of its first operand with the even rows of its
// second, resp. the upper 32 lanes of the first with the lower 32 of the
// second), so that the epilogue waits on no LDS round trip.
// x of lane ^ 48 for lane groups 1 and 2 (rows 1 and 2 trade places); the
// result is unspecified in groups 0 and 3.
__device__ __forceinline__ int swap_rows12(int x, int g) {
  const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  // h[0] rows: x0 x1 x0 x1; h[1] rows: x2 x3 x2 x3
  const auto q = __builtin_amdgcn_permlane16_swap((uint32_t)h[0], (uint32_t)h[1], false, false);
  // q[0] rows: x0 x2 x0 x2; q[1] rows: x1 x3 x1 x3
  return (int)(g == 1 ? q[0] : q[1]);
}

// Scale operand of the P~ B operand.  FP6/FP4: the lane's own block.  FP8:
// lane group c supplies the scale of key block c; blocks 0/2 are the low/high
// halves held by groups 0-1, blocks 1/3 those held by groups 2-3, so groups
// 1 and 2 take the value from the lane 48 apart (a branch-free exchange).
template <int BITS>
__device__ __forceinline__ int p_scale(int s_lo, int s_hi, int g) {
  if (BITS != 8) return s_lo;
  const int give = g >= 2 ? s_lo : s_hi;            // what the partner needs
  const int got = swap_rows12(give, g);
  const int own = g < 2 ? s_lo : s_hi;
  const bool cross = (g == 1) | (g == 2);
  return cross ? got : own;
}

// The lane's Q' operand of the score product, MX-quantised here from the
// bf16 row (the same rule as the quantiser: OCP floor scale, RNE, saturation,
// NaN/Inf blocks get scale 0xFF and zero codes) with Q' = fp32(q * mult).
// `row` is null for padding rows.  Returns the codes in operand order and
// sets `sc` to the E8M0 byte of the block this lane group scales, raised by
// 23 (2^23 rides on Q's scale; 255 stays NaN).
template <int F, int D>
__device__ __forceinline__ opv<F> q_operand(const uint16_t* row, float mult, int g, int& sc) {
  constexpr int BITS = Fmt<F>::bits;
  float v[32];
  bool bad_lo = false, bad_hi = false;
  // element k of the operand: FP6/FP4 column 32g + k; FP8 column 16g + k
  // (k < 16) and 64 + 16g + (k - 16)
  auto column = [&](int k) { return BITS == 8 ? (k < 16 ? 16 * g + k : 64 + 16 * g + k - 16) : 32 * g + k; };
#pragma unroll
  for (int c = 0; c < 4; ++c) {                      // four 8-element chunks
    const int col = column(8 * c);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row != nullptr && col < D) w = *reinterpret_cast<const uint4*>(row + col);
    const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = h[e] & 0xFFFF, hi = h[e] >> 16;
      const bool nan_inf = ((lo & 0x7F80) == 0x7F80) | ((hi & 0x7F80) == 0x7F80);
      if (c < 2) bad_lo |= nan_inf; else bad_hi |= nan_inf;
      v[8 * c + 2 * e] = bf16_bits_to_float(lo) * mult;
      v[8 * c + 2 * e + 1] = bf16_bits_to_float(hi) * mult;
    }
  }
  float a_lo = 0.0f, a_hi = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    a_lo = __builtin_fmaxf(a_lo, __builtin_fabsf(v[k]));
    a_hi = __builtin_fmaxf(a_hi, __builtin_fabsf(v[16 + k]));
  }
  if (BITS == 8) {
    // each MX block is two half blocks held by lanes 16 apart
    a_lo = __builtin_fmaxf(a_lo, __shfl_xor(a_lo, 16));
    a_hi = __builtin_fmaxf(a_hi, __shfl_xor(a_hi, 16));
    bad_lo |= __shfl_xor((int)bad_lo, 16) != 0;
    bad_hi |= __shfl_xor((int)bad_hi, 16) != 0;
  } else {
    a_lo = a_hi = __builtin_fmaxf(a_lo, a_hi);
    bad_lo = bad_hi = bad_lo | bad_hi;
  }
  auto scale_exp = [](float amax) {
    int X = amax > 0.0f ? floor_log2(amax) - Fmt<F>::emax : -127;
    return X < -127 ? -127 : (X > 127 ? 127 : X);
  };
  const int x_lo = scale_exp(a_lo), x_hi = scale_exp(a_hi);
  float y[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) y[k] = __builtin_ldexpf(v[k], -(k < 16 ? x_lo : x_hi));
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  Pack32<F, true>::run(y, w);
  if (bad_lo) { for (int i = 0; i < 4; ++i) w[i] = 0; }
  if (bad_hi) { for (int i = 4; i < 8; ++i) w[i] = 0; }
  if (BITS != 8 && bad_lo) { for (int i = 0; i < 8; ++i) w[i] = 0; }
  auto raised = [](int x, bool bad) { return bad ? 255 : min(x + 127 + 23, 254); };
  int s_lo = raised(x_lo, bad_lo), s_hi = raised(x_hi, bad_hi);
  if (BITS == 8 && D < 128) s_hi = 127;                // blocks past D: zeros
  if (BITS != 8 && 32 * g >= D) s_lo = s_hi = 127;
  sc = p_scale<BITS>(s_lo, s_hi, g);
  opv<F> o;
#pragma unroll
  for (int i = 0; i < Operand<F>::words; ++i) o[i] = (int)w[i];
  return o;
}

}  // namespace

template <int F, int D, bool CAUSAL, int NSUB, int NWAVES>
__global__ void __attribute__((amdgpu_flat_work_group_size(NWAVES * 64, NWAVES * 64), amdgpu_waves_per_eu(FSA_WPE))) fsa_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource types exist only in the device pass
  constexpr int BITS = Fmt<F>::bits;
  constexpr int MB = Fmt<F>::mbits;
  constexpr int PL = F == FMT_E4M3 ? Fmt<F>::emax - 1 : Fmt<F>::emax;   // placement binade
  constexpr int CAP = 127 - PL;
  constexpr int RB = D * BITS / 8;          // bytes per Q^/K^ row (global)
  constexpr int RS = 128;                   // bytes per K^/V^T row (LDS)
  constexpr int NCH = RS / 16;              // 16-byte chunks per LDS row
  constexpr int KCH_VALID = RB / 16 > 0 ? RB / 16 : 1;
  constexpr int VCH_VALID = KT * BITS / 8 / 16;
  constexpr int VRB = KT * BITS / 8;        // bytes per V^T tile row (global)
  constexpr int NDB = D / 32;               // MX blocks per Q^/K^ row
  constexpr int NDT = D / 16;               // 16-wide output tiles along D
  constexpr int QW = NWAVES * 16 * NSUB;    // queries per workgroup
  constexpr int K_BYTES = KT * RS;
  constexpr int V_BYTES = D * RS;
  constexpr int KS_BYTES = KT * NDB;
  constexpr int VS_BYTES = D * 4;
  constexpr int KSTAGE = K_BYTES + KS_BYTES;   // K^ tile and its scales
  constexpr int VSTAGE = V_BYTES + VS_BYTES;   // V^T tile and its scales

  // Block levels (a block's binade plus 127 + REF) between which the block
  // shifts are linear: at XLO and below the shift is CAP, at XHI and above
  // it is -EXT.
  constexpr int XLO = 127 + REF - CAP, XHI = 127 + REF + EXT;
  // Three-stage LDS rings, K^ and V^T each.  One LDS object per stage,
  // always addressed through a compile-time stage index: the compiler then
  // sees that reads of one stage cannot alias the DMA in flight into
  // another, and does not wait for that DMA first.
  // Ring depth: three stages for one workgroup per CU; two let two
  // workgroups share a CU (their barriers are independent).
  constexpr int NST = NWAVES == 8 ? 3 : 2;
  __shared__ __align__(16) uint8_t kl0[KSTAGE];
  __shared__ __align__(16) uint8_t kl1[KSTAGE];
  __shared__ __align__(16) uint8_t kl2[NST > 2 ? KSTAGE : 16];
  __shared__ __align__(16) uint8_t vl0[VSTAGE];
  __shared__ __align__(16) uint8_t vl1[VSTAGE];
  __shared__ __align__(16) uint8_t vl2[NST > 2 ? VSTAGE : 16];
  auto kstage = [&](auto st_tag) __attribute__((always_inline)) -> uint8_t* {
    constexpr int ST = decltype(st_tag)::value;
    if constexpr (ST == 0) return kl0;
    else if constexpr (ST == 1) return kl1;
    else return kl2;
  };
  auto vstage = [&](auto st_tag) __attribute__((always_inline)) -> uint8_t* {
    constexpr int ST = decltype(st_tag)::value;
    if constexpr (ST == 0) return vl0;
    else if constexpr (ST == 1) return vl1;
    else return vl2;
  };

  const int tid = threadIdx.x;
  // wave-uniform by construction; made scalar so that everything derived
  // from it (LDS DMA targets in particular) stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r = lane & 15;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of (head, query tile) work items so that the workgroups
  // sharing one XCD's L2 work on the same head's K^ and V^.
  const int nq = (a.S + QW - 1) / QW;
  const int n_items = nq * a.B * a.hrun;
  const int per_xcd = (n_items + 7) / 8;
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  // workspace slabs are indexed by the launch's own (batch, head) order;
  // outputs by the global head index
  const int64_t wi = item / nq;
  const int b = (int)wi / a.hrun;
  const int h = a.h0 + ((int)wi - b * a.hrun);
  const int64_t bh = (int64_t)b * a.H + h;
  const int S = a.S;
  const int q_wg = (item - (int)wi * nq) * QW;
  const int q_wave = q_wg + wave * 16 * NSUB;

  const uint8_t* kc = a.kc + wi * (int64_t)a.sk_alloc * RB;
  const uint8_t* ks = a.ks + wi * (int64_t)a.sk_alloc * NDB;
  const int64_t v_row = (int64_t)a.sk_alloc * BITS / 8;
  const uint8_t* vc = a.vc + wi * (int64_t)D * v_row;
  const int vs_row = a.sk_alloc / 32;
  const uint8_t* vs = a.vs + wi * (int64_t)D * vs_row;

  int n_tiles = (S + KT - 1) / KT;
  if (CAUSAL) {
    const int last_q = q_wg + QW - 1 < S - 1 ? q_wg + QW - 1 : S - 1;
    const int t_need = last_q / KT + 1;
    n_tiles = t_need < n_tiles ? t_need : n_tiles;
  }

  // Direct global->LDS copy of key tile t into stage st with buffer loads:
  // each wave moves 1 KB per instruction (8 LDS rows of 8 chunks); lane i
  // fills physical chunk i%8 of row i/8 with the logical chunk the swizzle
  // maps there (unused chunks of FP6/FP4 rows re-read chunk 0 of their row).
  // The lane's byte offset inside the head's slab is fixed for the whole
  // sweep; the tile's offset goes in the scalar offset, so issuing a tile
  // costs no vector instructions.
  constexpr int NK_DMA = KT * NCH / 64 / NWAVES;      // per wave, per tile
  constexpr int NV_DMA = D * NCH / 64 / NWAVES;
  constexpr int NKS = KS_BYTES / 256;                 // scale dwords per lane and tile
  constexpr int NVS = VS_BYTES / 256;
  static_assert(NKS <= NWAVES && NVS <= NWAVES, "one scale dword per wave");
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kc, (short)0, a.sk_alloc * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vc, (short)0, (int)(D * v_row), 0x00020000);
  const __amdgpu_buffer_rsrc_t ks_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)ks, (short)0, a.sk_alloc * NDB, 0x00020000);
  const __amdgpu_buffer_rsrc_t vs_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vs, (short)0, D * vs_row, 0x00020000);
  // The rows a wave fills are 8 * NWAVES apart; when that is a multiple of
  // the swizzle's period their swizzles agree, so one lane offset serves
  // them all and the row step goes into the scalar offset (fewer vector
  // registers held across the sweep).  Otherwise each row keeps its own lane
  // offset.
  constexpr int K_SWZ_PERIOD = D != 128 ? 1 : (BITS == 8 ? 32 : (BITS == 6 ? 128 : 64));   // rows
  constexpr int V_SWZ_PERIOD = BITS == 6 ? 16 : 8;
  constexpr bool ONE_KOFF = (8 * NWAVES) % K_SWZ_PERIOD == 0;
  constexpr bool ONE_VOFF = (8 * NWAVES) % V_SWZ_PERIOD == 0;
  constexpr int NKV = ONE_KOFF ? 1 : NK_DMA;
  constexpr int NVV = ONE_VOFF ? 1 : NV_DMA;
  // With one lane offset per operand the offsets are recomputed at every
  // issue from an opaque lane index (a few vector instructions) instead of
  // being held across the sweep, where the register allocator would rather
  // spill them, and reloading a spill would wait for the DMA in flight.
  auto k_lane_off = [&](int k, int ln) __attribute__((always_inline)) {
    const int row = (wave + NWAVES * k) * 8 + (ln >> 3);
    const int c = (ln & 7) ^ swz_k<F, D>(row);
    return row * RB + (c < KCH_VALID ? c : 0) * 16;
  };
  auto v_lane_off = [&](int k, int ln) __attribute__((always_inline)) {
    const int row = (wave + NWAVES * k) * 8 + (ln >> 3);
    const int c = (ln & 7) ^ swz_v<F>(row);
    return row * (int)v_row + (c < VCH_VALID ? c : 0) * 16;
  };
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int l = lane;
    if constexpr (ONE_KOFF || ONE_VOFF) asm volatile("" : "+v"(l));
    return l;
  };
  int k_voff[NKV], v_voff[NVV];
#pragma unroll
  for (int k = 0; k < NKV; ++k) k_voff[k] = k_lane_off(k, lane);
#pragma unroll
  for (int k = 0; k < NVV; ++k) v_voff[k] = v_lane_off(k, lane);
  // Scales are tile-ordered, 128 * D/32 (K^) and 4 * D (V^T) contiguous
  // bytes per tile: NKS resp. NVS dwords per lane, one per wave; the other
  // waves re-load the first dword (the same bytes to the same place) so that
  // every wave issues the same number of loads.  The wave's part goes in
  // the scalar offset.
  const int s_voff = lane * 4;
  // The wave index is made opaque at every issue so that the LDS targets
  // (one per stage and row group) are recomputed with a scalar add rather
  // than held in scalar registers across the sweep, where they would spill.
  auto opaque_wave = [&]() __attribute__((always_inline)) {
    int w = wave;
    asm volatile("" : "+s"(w));
    return w;
  };
  auto issue_k = [&](int t, uint8_t* base) __attribute__((always_inline)) {
    const int ln = opaque_lane();
    const int wv = opaque_wave();
    const int kv0 = ONE_KOFF ? k_lane_off(0, ln) : 0;
    const uint32_t lb = lds_addr(base);
    const int ks_soff = wv < NKS ? wv * 256 : 0;
#pragma unroll
    for (int k = 0; k < NK_DMA; ++k)
      dma_lds16(k_rsrc, lb + (wv + NWAVES * k) * 1024, ONE_KOFF ? kv0 : k_voff[k],
                t * KT * RB + (ONE_KOFF ? k * NWAVES * 8 * RB : 0));
    dma_lds4(ks_rsrc, lb + K_BYTES + ks_soff, ONE_KOFF ? ln * 4 : s_voff, t * KS_BYTES + ks_soff);
  };
  auto issue_v = [&](int t, uint8_t* base) __attribute__((always_inline)) {
    const int ln = opaque_lane();
    const int wv = opaque_wave();
    const int vv0 = ONE_VOFF ? v_lane_off(0, ln) : 0;
    const uint32_t lb = lds_addr(base);
    const int vs_soff = wv < NVS ? wv * 256 : 0;
#pragma unroll
    for (int k = 0; k < NV_DMA; ++k)
      dma_lds16(v_rsrc, lb + (wv + NWAVES * k) * 1024, ONE_VOFF ? vv0 : v_voff[k],
                t * VRB + (ONE_VOFF ? k * NWAVES * 8 * (int)v_row : 0));
    dma_lds4(vs_rsrc, lb + V_BYTES + vs_soff, ONE_VOFF ? ln * 4 : s_voff, t * VS_BYTES + vs_soff);
  };
  // DMA instructions each wave issues per K^ tile and per V^T tile
  constexpr int DMA_K = NK_DMA + 1;
  constexpr int DMA_V = NV_DMA + 1;

  if (n_tiles > 0) {
    issue_k(0, kl0);
    issue_v(0, vl0);
  }

  // ---- Q^ fragments (B operand of the score product), one per subtile
  opv<F> qf[NSUB];
  int qsc[NSUB];
  // quantised here from the bf16 rows; 2^23 rides on Q's E8M0 scale, so the
  // product is 2^23 s: the exponent-field units of the exponential
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q_wave + 16 * s + r;
    qf[s] = q_operand<F, D>(q < S ? a.q + (bh * S + q) * (int64_t)D : nullptr, a.qmul, g, qsc[s]);
  }

  // A operand of the score product for 16-key slice j of the tile in stage
  // st: row R of the slice is key kpos(R/4, 4j + R%4), so that output row
  // 4g+i lands on the lane's operand position 4j+i.
  auto k_frag = [&](int j, int& sc) __attribute__((always_inline)) -> opv<F> {
    const int kk = kpos<F>(r >> 2, 4 * j + (r & 3));
    const uint8_t* base = kl0;
    sc = g < NDB ? (int)base[K_BYTES + (r * NDB + g) * 8 + j] : 127;
    return lds_operand<F>(base + kk * RS, swz_k<F, D>(kk), g, D);
  };

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- frozen max from the first tile (keys [0, 128))
  float mg[NSUB];
  wait_dma();
  __syncthreads();
  // the rings fill ahead of the sweep
  if (n_tiles > 1) { issue_k(1, kl1); issue_v(1, vl1); }
  if (NST > 2 && n_tiles > 2) { issue_k(2, kl2); issue_v(2, vl2); }
  {
    v4f acc[NSUB][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int sc;
      const opv<F> kf = k_frag(j, sc);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[s][j] = mfma<F>(kf, qf[s], zero4, sc, qsc[s]);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int q = q_wave + 16 * s + r;
      float sum = 0.f, mx = -INFINITY;
      int cnt = 0;
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int key = kpos<F>(g, p);
        const bool vis = key < S && (!CAUSAL || key <= q);
        const float x = acc[s][p >> 2][p & 3];
        sum += vis ? x : 0.f;
        mx = vis ? __builtin_fmaxf(mx, x) : mx;
        cnt += vis ? 1 : 0;
      }
      sum += __shfl_xor(sum, 16); sum += __shfl_xor(sum, 32);
      cnt += __shfl_xor(cnt, 16); cnt += __shfl_xor(cnt, 32);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16)); mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const float mean = sum / (float)(cnt > 0 ? cnt : 1);
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int key = kpos<F>(g, p);
        const bool vis = key < S && (!CAUSAL || key <= q);
        const float dlt = acc[s][p >> 2][p & 3] - mean;
        ss += vis ? dlt * dlt : 0.f;
      }
      ss += __shfl_xor(ss, 16); ss += __shfl_xor(ss, 32);
      const float sd = __builtin_sqrtf(ss / (float)(cnt > 0 ? cnt : 1));
      const int nvis = CAUSAL ? (q + 1 < S ? q + 1 : S) : S;
      const float z = __builtin_sqrtf(2.0f * __builtin_logf((float)nvis)) + 1.0f;
      // statistics of 2^23 s, back to binades (exact power-of-two scaling)
      mg[s] = __builtin_fmaxf(mx, mean + z * sd) * 0x1p-23f + a.bias;
    }
  }

  // ---- main sweep
  // A block whose largest score exceeds the guess by e_b > 0 binades keeps
  // its codes and takes an E8M0 scale 2^e_b above the guess's: exactly the
  // row the oracle re-bases by kappa = max e_b, scaled by 2^kappa in both
  // O and l.  Only a row beyond EXT binades (scale bytes or fp32 sums could
  // overflow) is recomputed by the fallback kernel with the re-basing made
  // explicit.
  v4f O[NSUB][NDT];
  v4f L[NSUB];
  int kmax[NSUB];
  float c0s[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    L[s] = zero4;
    kmax[s] = -1000000;
    // accumulator start: fp32(2^23 (127 + R) - 2^23 m~), one rounding
    c0s[s] = __builtin_fmaf(-8388608.0f, mg[s], 8388608.0f * (127 + REF));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[s][dt] = zero4;
  }
  // The score products start from the 4-register quad {c0, c0, c0, c0}.
  // Where registers are tightest (FP8, two subtiles) the quads are rebuilt
  // at every tile (4 moves each) from the one value kept across the sweep.
  constexpr bool QUAD_PER_TILE = BITS == 8 && NSUB >= 2;
  v4f minit[NSUB];
  auto refresh_start = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      float c = c0s[s];
      if constexpr (QUAD_PER_TILE) asm volatile("" : "+v"(c));
      minit[s] = v4f{c, c, c, c};
    }
  };
  refresh_start();
  const v4i ones = ones_fp4();

  // Lane-constant LDS byte offsets.  For slice j of the score product the
  // lane's K^ row is kk0 + 4j (+48 for the FP8 high half), and its swizzle
  // does not depend on j; V^T row 16dt + r likewise.
  const int kk0 = BITS == 8 ? 16 * (r >> 2) + (r & 3) : 32 * (r >> 2) + (r & 3);
  const int ksw = swz_k<F, D>(kk0);
  const int vsw = swz_v<F>(r);
  constexpr int NOFF = BITS == 8 ? 2 : (BITS == 6 ? 3 : 1);   // row pieces per operand
  int k_off[NOFF], v_off[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    int lo;
    if (BITS == 8) lo = i == 0 ? 16 * g : 64 + 16 * g;
    else if (BITS == 6) lo = 24 * g + 8 * i;
    else lo = 16 * g;
    k_off[i] = kk0 * RS + 16 * ((lo >> 4) ^ ksw) + (lo & 15);      // in a K^ stage
    v_off[i] = r * RS + 16 * ((lo >> 4) ^ vsw) + (lo & 15);         // in a V^T stage
  }
  // Scale bytes of the lane's 8 score products (slice j) and 8 P V products
  // (output tile dt), tile-ordered so that one read fetches all of them; the
  // MFMA selects byte j & 3 / dt & 3 of a dword.  Lanes past D (D = 64)
  // multiply zeros and take scale 1.
  const int ks_off = K_BYTES + (r * NDB + (g < NDB ? g : 0)) * 8;
  const int vs_off = V_BYTES + (r * 4 + g) * NDT;
  auto k_scales = [&](const uint8_t* base) __attribute__((always_inline)) -> uint2 {
    const uint2 v = *reinterpret_cast<const uint2*>(base + ks_off);
    return g < NDB ? v : make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  };
  auto v_scales = [&](const uint8_t* base) __attribute__((always_inline)) -> uint2 {
    if constexpr (NDT == 8) return *reinterpret_cast<const uint2*>(base + vs_off);
    else return make_uint2(*reinterpret_cast<const uint32_t*>(base + vs_off), 0u);
  };
  // Fragments in flight per operand stream: 0 leaves the order to the
  // compiler (with the FP6 slice fence); FP8 reads three ahead in a fixed
  // order (measured best; left free, the compiler hoists every read of a
  // phase and runs out of registers).
  constexpr int PIPE = FSA_PIPE >= 0 ? FSA_PIPE : (BITS == 8 ? 3 : 0);
  const bool k_live = 32 * g < D;               // FP6/FP4 lane groups past D
  const bool k_hi = 64 + 16 * g < D;            // FP8 high half present

  // Fragment reads go through the stage object itself (never an opaque
  // address): the compiler then knows which stage a read touches and does
  // not make it wait for the DMA in flight into the others.
  struct Rows { const uint8_t* base; const int* off; };
  auto rows = [&](const uint8_t* stage, const int* off) __attribute__((always_inline)) -> Rows {
    return Rows{stage, off};
  };
  auto frag = [&](const Rows& rw, int imm, bool live, bool hi) __attribute__((always_inline)) -> opv<F> {
    opv<F> o = zero_operand<F>();
    const uint8_t* base = rw.base;
    const int* off = rw.off;
    if constexpr (BITS == 8) {
      if (live) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(base + off[0] + imm);
        o[0] = a0.x; o[1] = a0.y; o[2] = a0.z; o[3] = a0.w;
      }
      if (hi) {
        const uint4 a1 = *reinterpret_cast<const uint4*>(base + off[1] + imm);
        o[4] = a1.x; o[5] = a1.y; o[6] = a1.z; o[7] = a1.w;
      }
    } else if constexpr (BITS == 6) {
      if (live) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const uint2 a = *reinterpret_cast<const uint2*>(base + off[i] + imm);
          o[2 * i] = a.x; o[2 * i + 1] = a.y;
        }
      }
    } else if (live) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(base + off[0] + imm);
      o[0] = a0.x; o[1] = a0.y; o[2] = a0.z; o[3] = a0.w;
    }
    return o;
  };
  // K^ fragment of 16-key slice j; V^T fragment of output tile dt
  auto kfrag = [&](const Rows& rw, int j) __attribute__((always_inline)) -> opv<F> {
    const int jrow = 4 * j + ((BITS == 8 && j >= 4) ? 48 : 0);
    return frag(rw, jrow * RS, BITS == 8 ? 16 * g < D : k_live, BITS == 8 ? k_hi : false);
  };
  auto vfrag = [&](const Rows& rw, int dt) __attribute__((always_inline)) -> opv<F> {
    return frag(rw, 16 * dt * RS, true, true);
  };

  // FP6 fragments arrive in three 8-byte pieces per lane; left free, the
  // scheduler hoists them for many slices at once and pays in register
  // copies.  A scheduling fence after each slice's MFMAs keeps FP6 loads
  // next to their use (measured: about +20 % for E2M3, a loss for the others).
  auto slice_fence = [&]() __attribute__((always_inline)) {
    if constexpr (BITS == 6) __builtin_amdgcn_sched_barrier(0);
  };

  // State of one key tile: the score accumulators of each subtile, and P~ of
  // each subtile in operand form with its scale byte.
  v4f acc[NSUB][8];
  opv<F> pw[NSUB];
  int psc[NSUB];

  // Scores of the tile in stage `base`: y = 2^23 s + accumulator start.  In
  // a masked tile the accumulator of an invisible key starts at -inf, so its
  // y is -inf and its pattern 0: the epilogue carries no masking at all.
  auto qk_into = [&](const uint8_t* base, int key0, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if constexpr (QUAD_PER_TILE) refresh_start();
    if constexpr (MASKED) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int q = q_wave + 16 * s + r;
        const int lim = CAUSAL ? min(S, q + 1) : S;     // keys [0, lim) visible
#pragma unroll
        for (int p = 0; p < 32; ++p)
          acc[s][p >> 2][p & 3] = key0 + kpos<F>(g, p) < lim ? c0s[s] : -INFINITY;
      }
    }
    const uint2 ksc = k_scales(base);
    const Rows rw = rows(base, k_off);
    if constexpr (PIPE > 0) {
      // PIPE fragments in flight: the read of slice j+PIPE issues right
      // after the products of slice j, in a fixed order
      opv<F> kfs[PIPE > 0 ? PIPE : 1];
#pragma unroll
      for (int j = 0; j < PIPE; ++j) kfs[j] = kfrag(rw, j);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          acc[s][j] = mfma_sel<F>(kfs[j % PIPE], qf[s], MASKED ? acc[s][j] : minit[s],
                                  (int)(j < 4 ? ksc.x : ksc.y), j, qsc[s]);
        if (j + PIPE < 8) kfs[j % PIPE] = kfrag(rw, j + PIPE);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const opv<F> kf = kfrag(rw, j);
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          acc[s][j] = mfma_sel<F>(kf, qf[s], MASKED ? acc[s][j] : minit[s],
                                  (int)(j < 4 ? ksc.x : ksc.y), j, qsc[s]);
        slice_fence();
      }
    }
  };

  // Fused exponential + MX quantisation of P for the scores of subtile s.
  //
  // The bit-pattern exponential: y's integer part is the fp32 pattern of
  // 2^(t + R).  It is monotone in y, and exact wherever y >= 2^24 (below, the
  // block sits beyond the largest shift anyway), so the block maxima are
  // taken on the integers, and y is dead once converted.
  auto epi_sub = [&](int s) __attribute__((always_inline)) {
    // patterns in the operand order of the pack conversion: FP6 takes even
    // and odd elements as two 16-register sources
    float pv[32];
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      const int o = BITS == 6 ? (p & 1) * 16 + (p >> 1) : p;
      pv[o] = __uint_as_float(cvt_u32_trunc(acc[s][p >> 2][p & 3]));
    }
    auto u = [&](int o) __attribute__((always_inline)) { return __float_as_uint(pv[o]); };
    // maxima of the two halves of the lane's 32 values
    uint32_t m0 = max(max(u(0), u(1)), u(2));
    uint32_t m1 = max(max(u(16), u(17)), u(18));
#pragma unroll
    for (int p = 3; p < 15; p += 2) {
      m0 = max(max(m0, u(p)), u(p + 1));
      m1 = max(max(m1, u(16 + p)), u(17 + p));
    }
    m0 = max(m0, u(15));
    m1 = max(m1, u(31));
    // One block maximum per lane.  FP6/FP4: the lane's own block.  FP8: a
    // lane holds half blocks; one swap of the two half maxima across the
    // 16-lane rows completes one whole block per lane group, group g ending
    // up with block (0, 2, 1, 3)[g].
    uint32_t mb;
    if constexpr (BITS == 8) {
      const auto h = __builtin_amdgcn_permlane16_swap(m0, m1, false, false);
      mb = max((uint32_t)h[0], (uint32_t)h[1]);
    } else {
      mb = max(m0, m1);
    }
    const int x = block_level<MB>(mb);
    kmax[s] = max(kmax[s], x);
    // scale byte 127 - pl - d of that block (d = the block shift); the
    // conversion divides by 2^(sb + R - 127) = 2^(R - pl - d)
    const int sb = min(max(x, XLO), XHI) - REF - PL;
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (BITS == 8) {
      // the lane's low and high half blocks, then block g for the B scale
      const auto hl = __builtin_amdgcn_permlane16_swap((uint32_t)sb, (uint32_t)sb, false, false);
      const int sb_lo = (int)hl[0], sb_hi = (int)hl[1];
      Pack32<F, false>::run(pv, w, conv_scale(sb_lo), conv_scale(sb_hi));
      const auto hd = __builtin_amdgcn_permlane32_swap((uint32_t)sb_lo, (uint32_t)sb_hi, false, false);
      psc[s] = (int)((g & 1) ? hd[1] : hd[0]);
    } else {
      if constexpr (BITS == 6) pack_fp6_split(pv, w, conv_scale(sb));
      else Pack32<F, false>::run(pv, w, conv_scale(sb), conv_scale(sb));
      psc[s] = sb;
    }
#pragma unroll
    for (int i = 0; i < Operand<F>::words; ++i) pw[s][i] = (int)w[i];
  };

  // P V and the row sums on the matrix cores, V^T tile in stage `base`.
  auto pv_step = [&](const uint8_t* base) __attribute__((always_inline)) {
    const uint2 vsc = v_scales(base);
    const Rows rw = rows(base, v_off);
    if constexpr (PIPE > 0) {
      opv<F> vfp[PIPE > 0 ? PIPE : 1];
#pragma unroll
      for (int dt = 0; dt < PIPE && dt < NDT; ++dt) vfp[dt] = vfrag(rw, dt);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          O[s][dt] = mfma_sel<F>(vfp[dt % PIPE], pw[s], O[s][dt], (int)(dt < 4 ? vsc.x : vsc.y), dt, psc[s]);
        if (dt + PIPE < NDT) vfp[dt % PIPE] = vfrag(rw, dt + PIPE);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const opv<F> vf = vfrag(rw, dt);
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          O[s][dt] = mfma_sel<F>(vf, pw[s], O[s][dt], (int)(dt < 4 ? vsc.x : vsc.y), dt, psc[s]);
        slice_fence();
      }
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) L[s] = row_sum<F>(ones, pw[s], L[s], psc[s]);
  };

  // tiles [0, n_clean) need no masking for any row of this wave
  int n_clean = S / KT;
  if (CAUSAL) {
    const int c2 = (q_wave + 1) / KT;          // key0 + KT - 1 <= q_wave
    n_clean = c2 < n_clean ? c2 : n_clean;
  }
  n_clean = n_clean < n_tiles ? n_clean : n_tiles;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  if constexpr (NST == 2) {
    // Two stages: tile t+1 lands while tile t is read; after the barrier
    // that ends step t its stages take tile t+2.
    auto step2 = [&](int t, auto st_tag) __attribute__((always_inline)) {
      uint8_t* kb = kstage(st_tag);
      uint8_t* vb = vstage(st_tag);
      if (t < n_clean) qk_into(kb, t * KT, std::false_type{});
      else qk_into(kb, t * KT, std::true_type{});
#pragma unroll
      for (int s = 0; s < NSUB; ++s) epi_sub(s);
      if constexpr (PIPE > 0) __builtin_amdgcn_sched_barrier(0);
      pv_step(vb);
      wait_dma();
      ring_barrier();
      if (t + 2 < n_tiles) {
        issue_k(t + 2, kb);
        issue_v(t + 2, vb);
      }
    };
    for (int t = 0; t < n_tiles; t += 2) {
      step2(t, I0{});
      if (t + 1 < n_tiles) step2(t + 1, I1{});
    }
  } else {
  // Tile after tile, one barrier per tile; two waves per SIMD overlap one's
    // vector epilogue with the other's products.  Tile t+1 must have landed
    // by the end of step t (t+2 may still be in flight); after the barrier the
    // stages of tile t take tile t+3.  FP8 issues the loads of a tile in two
    // halves (measured a little faster; a little slower for FP6/FP4): K^ tile
    // t+3 right after the barrier that ends step t, V^T tile t+2 after the
    // score products of step t (into the stage of tile t-1, free since the
    // barrier that ended step t-1).  Either way the loads of tile t+1 precede
    // those of tile t+2 in issue order, so the count kept in flight stays one
    // tile.
    constexpr bool SPLIT = BITS == 8;
    auto step = [&](int t, auto st_tag) __attribute__((always_inline)) {
      constexpr int P = decltype(st_tag)::value;
      uint8_t* kb = kstage(st_tag);
      uint8_t* vb = vstage(st_tag);
      if (t < n_clean) qk_into(kb, t * KT, std::false_type{});
      else qk_into(kb, t * KT, std::true_type{});
      if (SPLIT && t >= 1 && t + 2 < n_tiles)
        issue_v(t + 2, vstage(std::integral_constant<int, (P + 2) % 3>{}));
#pragma unroll
      for (int s = 0; s < NSUB; ++s) epi_sub(s);
      // keep the P V fragment reads below the epilogue: hoisted above it they
      // would hold registers through it
      if constexpr (PIPE > 0) __builtin_amdgcn_sched_barrier(0);
      pv_step(vb);
      if (t + 2 < n_tiles) wait_dma_keep<DMA_K + DMA_V>();
      else wait_dma();
      ring_barrier();
      if (t + 3 < n_tiles) {
        issue_k(t + 3, kb);
        if (!SPLIT) issue_v(t + 3, vb);
      }
    };
    for (int t = 0; t < n_tiles; t += 3) {
      step(t, I0{});
      if (t + 1 < n_tiles) step(t + 1, I1{});
      if (t + 2 < n_tiles) step(t + 2, I2{});
    }
  }

  // row offsets in binades (the oracle's kappa); rows beyond EXT come out
  // wrong here and are recomputed by the fallback kernel
  int kap[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    int k = kmax[s] - (127 + REF);            // block level -> binade
    k = max(k, __shfl_xor(k, 16));
    k = max(k, __shfl_xor(k, 32));
    kap[s] = k > 0 ? k : 0;
  }

  // ---- normalise and store: lane (g, r) holds O[q][16dt + 4g + i]
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q_wave + 16 * s + r;
    if (q < S) {
      const float inv = 1.0f / L[s][0];
      uint16_t* orow = a.out + (bh * S + q) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t lo = f32_to_bf16_rne(O[s][dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(O[s][dt][1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_rne(O[s][dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(O[s][dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
      if (g == 0) {
        a.row_kappa[bh * S + q] = kap[s];
        a.row_mguess[bh * S + q] = mg[s];
      }
    }
  }
  // tell the fallback kernel of this call that it has work (one vector store)
  bool beyond = false;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) beyond |= kap[s] > EXT;
  if (__builtin_amdgcn_ballot_w64(beyond) != 0 && lane == 0) *a.fb_flag = a.call_id;
#endif  // __HIP_DEVICE_COMPILE__
}

// Fallback for rows whose scores exceed the frozen max by more than EXT
// binades: one wave per 32 query rows (two subtiles of 16).  A wave whose
// rows all stayed within EXT exits at once; otherwise it recomputes its rows
// from global memory with each row's reference raised by its kappa
// (accumulator start and block shifts re-based, no in-loop clamp), reading
// the frozen max and kappa the main kernel stored, and overwrites their
// outputs.  Rows within EXT come out as the main kernel left them (the
// re-based sums are the same up to the common power-of-two factor).  L32:
// the scales are in the *_TILES32 layouts of the 32x32x64 kernel.
template <int F, int D, bool CAUSAL, bool L32>
__device__ __forceinline__ void fallback_group(const AttnArgs& a, int64_t grp) {
  constexpr int NSUB = 2;
  constexpr int BITS = Fmt<F>::bits;
  constexpr int MB = Fmt<F>::mbits;
  constexpr int PL = F == FMT_E4M3 ? Fmt<F>::emax - 1 : Fmt<F>::emax;
  constexpr int CAP = 127 - PL;
  constexpr int RB = D * BITS / 8;
  constexpr int NDB = D / 32;
  constexpr int NDT = D / 16;
  constexpr int VRB = KT * BITS / 8;
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int S = a.S;
  const int ng = (S + 16 * NSUB - 1) / (16 * NSUB);
  const int64_t wi = grp / ng;
  if (wi >= (int64_t)a.B * a.hrun) return;
  const int b = (int)wi / a.hrun;
  const int h = a.h0 + ((int)wi - b * a.hrun);
  const int64_t bh = (int64_t)b * a.H + h;
  const int q0 = (int)(grp - wi * ng) * 16 * NSUB;

  int kap[NSUB];
  float mg[NSUB];
  bool extreme = false;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q0 + 16 * s + r;
    kap[s] = q < S ? a.row_kappa[bh * S + q] : 0;
    mg[s] = q < S ? a.row_mguess[bh * S + q] : 0.0f;
    extreme |= kap[s] > EXT;
  }
  if (__builtin_amdgcn_ballot_w64(extreme) == 0) return;

  const uint8_t* kc = a.kc + wi * (int64_t)a.sk_alloc * RB;
  const uint8_t* ks = a.ks + wi * (int64_t)a.sk_alloc * NDB;
  const int64_t v_row = (int64_t)a.sk_alloc * BITS / 8;
  const uint8_t* vc = a.vc + wi * (int64_t)D * v_row;
  const int vs_row = a.sk_alloc / 32;
  const uint8_t* vs = a.vs + wi * (int64_t)D * vs_row;
  // scale byte of tile key kk (read by lane (g, r) as slice j) and D block g
  auto ks_byte = [&](int kk, int j) __attribute__((always_inline)) {
    return L32 ? key_tile32_byte(kk, g, D, BITS) : (r * NDB + g) * 8 + j;
  };

  opv<F> qf[NSUB];
  int qsc[NSUB];
  v4f mk[NSUB], O[NSUB][NDT], L[NSUB];
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q0 + 16 * s + r;
    qf[s] = q_operand<F, D>(q < S ? a.q + (bh * S + q) * (int64_t)D : nullptr, a.qmul, g, qsc[s]);
    L[s] = zero4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[s][dt] = zero4;
  }
  const v4i ones = ones_fp4();

  int n_tiles = (S + KT - 1) / KT;
  if (CAUSAL) {
    const int last_q = q0 + 16 * NSUB - 1 < S - 1 ? q0 + 16 * NSUB - 1 : S - 1;
    n_tiles = min(n_tiles, last_q / KT + 1);
  }
  // The main sweep measures binades on the integer patterns, which saturate
  // some 320 binades above the guess; take kappa again from the fp32 values
  // (exact to HI_BINADE).
  {
    v4f m0init[NSUB];
    int km[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const float c0 = __builtin_fmaf(-8388608.0f, mg[s], 8388608.0f * (float)(127 + REF));
      m0init[s] = v4f{c0, c0, c0, c0};
      km[s] = -(1 << 30);
    }
    for (int t = 0; t < n_tiles; ++t) {
      const int key0 = t * KT;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = kpos<F>(r >> 2, 4 * j + (r & 3));
        const int sc = g < NDB ? (int)ks[(int64_t)t * KT * NDB + ks_byte(kk, j)] : 127;
        const opv<F> kf = global_operand<F>(kc + (int64_t)(key0 + kk) * RB, g, D);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const v4f y = mfma<F>(kf, qf[s], m0init[s], sc, qsc[s]);
          const int q = q0 + 16 * s + r;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + kpos<F>(g, 4 * j + i);
            const bool vis = key < S && (!CAUSAL || key <= q);
            // the binade of each element bounds that of its block's maximum
            if (vis) km[s] = max(km[s], block_binade<MB>(y[i]));
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      int k = km[s];
      k = max(k, __shfl_xor(k, 16));
      k = max(k, __shfl_xor(k, 32));
      kap[s] = k > 0 ? k : 0;
      const float c0 = __builtin_fmaf(-8388608.0f, mg[s], 8388608.0f * (float)(127 + REF - kap[s]));
      mk[s] = v4f{c0, c0, c0, c0};
      const int q = q0 + 16 * s + r;
      if (g == 0 && q < S) a.row_kappa[bh * S + q] = kap[s];
    }
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * KT;
    v4f acc[NSUB][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = kpos<F>(r >> 2, 4 * j + (r & 3));
      const int sc = g < NDB ? (int)ks[(int64_t)t * KT * NDB + ks_byte(kk, j)] : 127;
      const opv<F> kf = global_operand<F>(kc + (int64_t)(key0 + kk) * RB, g, D);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[s][j] = mfma<F>(kf, qf[s], mk[s], sc, qsc[s]);
    }
    opv<F> pw[NSUB];
    int psc[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int q = q0 + 16 * s + r;
      float x[32];
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int key = key0 + kpos<F>(g, p);
        const bool vis = key < S && (!CAUSAL || key <= q);
        x[p] = vis ? acc[s][p >> 2][p & 3] : -INFINITY;
      }
      float m0 = x[0], m1 = x[16];
#pragma unroll
      for (int p = 1; p < 16; ++p) { m0 = __builtin_fmaxf(m0, x[p]); m1 = __builtin_fmaxf(m1, x[16 + p]); }
      if (BITS == 8) {
        m0 = __builtin_fmaxf(m0, __shfl_xor(m0, 16));
        m1 = __builtin_fmaxf(m1, __shfl_xor(m1, 16));
      } else {
        m0 = __builtin_fmaxf(m0, m1);
        m1 = m0;
      }
      // binades relative to the raised reference: shifts need no EXT clamp
      const int sb0 = 127 - PL - min(-block_binade<MB>(m0), CAP);
      const int sb1 = 127 - PL - min(-block_binade<MB>(m1), CAP);
      float pv[32];
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int key = key0 + kpos<F>(g, p);
        const bool vis = key < S && (!CAUSAL || key <= q);
        const uint32_t u = cvt_u32_trunc(acc[s][p >> 2][p & 3]);
        pv[p] = __uint_as_float(vis ? u : 0u);
      }
      uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      Pack32<F, false>::run(pv, w, conv_scale(sb0), conv_scale(sb1));
#pragma unroll
      for (int i = 0; i < Operand<F>::words; ++i) pw[s][i] = (int)w[i];
      psc[s] = p_scale<BITS>(sb0, sb1, g);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = 16 * dt + r;
      const opv<F> vf = global_operand<F>(vc + d * v_row + (int64_t)t * VRB, g, KT);
      const int vsc = (int)vs[(int64_t)t * 4 * D + (L32 ? dim_tile32_byte(d, g, D) : (r * 4 + g) * NDT + dt)];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) O[s][dt] = mfma<F>(vf, pw[s], O[s][dt], vsc, psc[s]);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) L[s] = row_sum<F>(ones, pw[s], L[s], psc[s]);
  }

#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q0 + 16 * s + r;
    if (q < S) {
      const float inv = 1.0f / L[s][0];
      uint16_t* orow = a.out + (bh * S + q) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t lo = f32_to_bf16_rne(O[s][dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(O[s][dt][1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_rne(O[s][dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(O[s][dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
    }
  }
}

// Grid-stride over groups of 32 query rows; a call whose main kernel found
// no row beyond EXT binades (flag not stamped with this call's id) exits
// after one load.
template <int F, int D, bool CAUSAL, bool L32>
__global__ void __launch_bounds__(64) fsa_fallback_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (*a.fb_flag != a.call_id) return;
  const int64_t n_groups = (int64_t)(a.S + 31) / 32 * a.B * a.hrun;
  for (int64_t grp = blockIdx.x; grp < n_groups; grp += gridDim.x)
    fallback_group<F, D, CAUSAL, L32>(a, grp);
#endif  // __HIP_DEVICE_COMPILE__
}

// Query subtiles (16 rows each) per wave.  More subtiles reuse every K^/V^T
// fragment read from LDS for more rows; the count is capped by the 256
// architectural VGPRs the score accumulators and the epilogue need.
template <int F> struct Nsub;
template <> struct Nsub<FMT_E4M3> { static constexpr int value = FSA_NSUB8; };
template <> struct Nsub<FMT_E2M3> { static constexpr int value = FSA_NSUB6; };
template <> struct Nsub<FMT_E2M1> { static constexpr int value = FSA_NSUB4; };
// Waves per workgroup.  Four (one per SIMD) on two-stage rings lets two
// workgroups share a CU, two waves per SIMD whose barriers are independent
// (measured: +11 % for E2M1, +1-2 % for the others over eight waves of one
// workgroup on three-stage rings, which the code keeps as an option).  Every
// kernel is built for two waves per SIMD (at most 256 registers each).
template <int F> struct Nwaves;
template <> struct Nwaves<FMT_E4M3> { static constexpr int value = FSA_NW8; };
template <> struct Nwaves<FMT_E2M3> { static constexpr int value = FSA_NW6; };
template <> struct Nwaves<FMT_E2M1> { static constexpr int value = FSA_NW4; };

template <int F, int D, bool CAUSAL>
hipError_t launch3(const AttnArgs& a, hipStream_t stream) {
  constexpr int NSUB = Nsub<F>::value;
  constexpr int NWAVES = Nwaves<F>::value;
  constexpr int QW = NWAVES * 16 * NSUB;
  const int n_items = (a.S + QW - 1) / QW * a.B * a.hrun;
  dim3 grid((n_items + 7) / 8 * 8);
  hipLaunchKernelGGL((fsa_fwd_kernel<F, D, CAUSAL, NSUB, NWAVES>), grid, dim3(NWAVES * 64), 0, stream, a);
  const int n_groups = (a.S + 31) / 32 * a.B * a.hrun;
  hipLaunchKernelGGL((fsa_fallback_kernel<F, D, CAUSAL, false>), dim3(n_groups < 1024 ? n_groups : 1024),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int F>
hipError_t launch2(const AttnArgs& a, int D, int causal, hipStream_t stream) {
  if (D == 128) return causal ? launch3<F, 128, true>(a, stream) : launch3<F, 128, false>(a, stream);
  return causal ? launch3<F, 64, true>(a, stream) : launch3<F, 64, false>(a, stream);
}

}  // namespace fsa
