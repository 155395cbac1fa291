// Device helpers of the fused-softmax attention kernel (gfx950).
//
// What the path computes (Fused-Softmax for efficient quantized attention,
// summary; Moving softmax to matrix operations speeds up AI inference by over
// 2x, "Read it as" and the "How it works" figure; the exact readings are
// fixed in the oracle's module documentation):
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
//      rows beyond 64 binades are recomputed by a second, re-based pass
//      of the same kernel;
//   6. out = bf16(O / l).
#pragma once

#include <type_traits>

#include "fsa_device.h"
#include "fsa_internal.h"
#include "lds_dma.h"

namespace fsa {

// The builtin of the scaled MFMA only takes 8-dword operands; the narrow
// FP6/FP4 forms of the same intrinsic are reached through its overloaded
// LLVM name.  (Compiler instructions: the hazard handling is the same.)
__device__ v4f mfma_scale_v4(v4i a, v4i b, v4f c, int cbsz, int blgp, int opsel_a, int sa,
                             int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v4i32");
// Mixed widths: an FP4 A operand with an FP6 B operand.
__device__ v4f mfma_scale_v4_v6(v4i a, v6i b, v4f c, int cbsz, int blgp, int opsel_a, int sa,
                                int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v6i32");

// P~ variants (the epilogue's modes).  BLOCK: each 32-key block shifted to
// the placement binade (the default).  ROW: one scale per row (E4M3).  EFQ:
// codes by one affine rule in the code domain (E2M1; EFQ-Softmax:
// Exp-Free Quantization for Softmax, abstract).  EXP: the exact exponential
// (the vector unit's exp2) in place of the bit pattern, i.e. P~ rounded from
// 2^x itself: the rounding thresholds of the exact map.
enum { PM_BLOCK = 0, PM_ROW = 1, PM_EFQ = 2, PM_EXP = 3 };

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
// y = lo: 0 in the sweep, which already puts them beyond the largest block
// shift.  The fallback pass measures a row's score itself (y negative for a
// row more than 127 + REF binades below its guess) and passes a lower lo.
// The rounding is exact for negative y too: the integer bias shifts y by a
// whole number of binades, which rounding to nearest even commutes with.  Values
// more than HI_BINADE binades above the reference count as exactly that
// many (the MAGIC window holds 2^22 codes); the row then falls back with
// kappa = HI_BINADE, which is exact for every score within 2^18 binades of
// its frozen max.
constexpr int HI_BINADE = 1 << 18;
// Largest guess-relative block binade the main sweep absorbs by block shifts
// alone; rows above it go to the re-based fallback pass.
constexpr int EXT = 64;
// Largest lead of the frozen max over the row's window max, in binades.  A
// row's top score is at least its window max, so its top block lies at most
// GUESS_CAP + 1 binades below the guess: within the largest block shift
// (127 - pl >= 119 binades for every P~ format), so that only a positive
// guess bias can send a row of a block map to the downward fallback.
constexpr int GUESS_CAP = 64;
static_assert(GUESS_CAP + 1 < 127 - 8, "capped guesses must stay within the block shifts");
static_assert(HI_BINADE > EXT, "clamped binades must reach the fallback pass");
// Lowest offset the fallback pass measures: rows down to HI_BINADE binades
// below their guess (the frozen max can lie far above a row whose scores
// have a light upper tail) are measured exactly, as rows far above are.
constexpr float LO_PATTERN = -8388608.0f * (float)(HI_BINADE - 127 - REF);
template <int M>
__device__ __forceinline__ int block_binade(float y, float lo = 0.0f) {
  const float yc = __builtin_amdgcn_fmed3f(y, lo, 8388608.0f * (float)(127 + REF + HI_BINADE));
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

// Largest block level whose offset the first pass records exactly: the
// patterns themselves stay exact up to level 511 (y < 2^32); rows at
// KSAT binades or more above their guess are marked as KSAT and measured
// again by the fallback pass.
constexpr int LEVEL_MAX = 510;
constexpr int KSAT = LEVEL_MAX - (127 + REF);
static_assert(KSAT > EXT, "offsets beyond the in-sweep shifts must be recorded");

// Level of a block whose largest pattern is m: the binade plus 127 + REF,
// i.e. the exponent field of m after rounding its mantissa to M bits
// (nearest, ties to even): floor(RNE(2^M m / 2^23) / 2^M).  For a pattern
// from y >= 2^23 this is the binade of block_binade below; smaller patterns
// lie below every level the shifts distinguish.  m is clamped first so that
// the rounding cannot carry out of 32 bits; up to LEVEL_MAX the level is
// exact, so the first pass knows the offset of every row below KSAT.
template <int M>
__device__ __forceinline__ int block_level(uint32_t m) {
  constexpr uint32_t LIM = (uint32_t)LEVEL_MAX << 23;
  const uint32_t mc = min(m, LIM);
  const uint32_t lsb = (mc >> (23 - M)) & 1u;
  return (int)((mc + (1u << (22 - M)) - 1u + lsb) >> 23);
}

// Truncation toward zero to u32 (v_cvt_u32_f32, which saturates and maps NaN
// and negatives to 0; the exponential relies on that).  C++ leaves those
// cases undefined (LLVM: poison), so what holds is the instruction the
// backend emits for the plain conversion, and a host test checks that it
// stays one bare v_cvt_u32_f32.  llvm.fptoui.sat.i32.f32 states the
// saturation in IR, but this compiler lowers it with two compare/select
// pairs around the same instruction (four more vector instructions per
// score element).  It must stay a compiler-visible conversion: the epilogue
// feeds it straight from MFMA results, and only instructions the compiler
// sees get the wait states that reading an MFMA result requires.  Its input
// must come straight from the product (never a select with constants), so
// that no out-of-range case can be folded away at compile time; masking
// happens on the integer result.
__device__ __forceinline__ uint32_t cvt_u32_trunc(float y) {
  return (uint32_t)y;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

// Row sums l += 1 P~^T on the matrix core with an FP4 ones operand (E2M1
// 1.0 = 0x2 per nibble, 4 registers) against P~ in its own format: FP4 ones
// times P~ is the same exact sum.
template <int F>
__device__ __forceinline__ v4f row_sum(const v4i& ones, const opv<F>& p, const v4f& c, int sp) {
  static_assert(Fmt<F>::bits != 8, "FP8 row sums take the 32x32x64 product");
  if constexpr (Fmt<F>::bits == 6)
    return mfma_scale_v4_v6(ones, p, c, Fmt<FMT_E2M1>::mfma, Fmt<F>::mfma, 0, 127, 0, sp);
  else
    return mfma_scale_v4(ones, p, c, Fmt<FMT_E2M1>::mfma, Fmt<F>::mfma, 0, 127, 0, sp);
}

// Raw bf16 words of four 8-element pieces of a Q row, at columns col[0..3]
// (each inside the row: the callers' chunks lie below D).  The loads are
// unconditional, a padding row (valid false) reading a real row and zeroing
// what it got, so that the compiler issues every piece of every chunk
// before the first wait: branches around them made it wait for each load
// in turn (vmcnt(0), which also drains the tile DMA in flight).  The mask
// is opaque, or the compiler would move each load back under a branch.
__device__ __forceinline__ void q_words(const uint16_t* row, bool valid, const int (&col)[4],
                                        uint4 (&w)[4]) {
  uint32_t m = valid ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    const uint4 x = *reinterpret_cast<const uint4*>(row + col[ch]);
    w[ch] = make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
  }
}
// Columns of the pieces of MX block g of a Q row (FP6/FP4 operands).
__device__ __forceinline__ void q_cols(int g, int (&col)[4]) {
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) col[ch] = 32 * g + 8 * ch;
}

// The lane's Q' operand of the score product, MX-quantised here from the
// bf16 words of MX block g (q_words over q_cols(g); the same rule as the
// quantiser: OCP floor scale, RNE, saturation, NaN/Inf blocks get scale 0xFF
// and zero codes) with Q' = fp32(q * mult).  Returns the codes in operand
// order and sets `sc` to the E8M0 byte of the block this lane group scales,
// raised by RAISE (2^23 rides on Q's scale for the bit-pattern exponential;
// 255 stays NaN).
template <int F, int RAISE>
__device__ __forceinline__ opv<F> q_operand(const uint4 (&qw)[4], float mult, int& sc) {
  static_assert(Fmt<F>::bits != 8, "FP8 Q' operands: q_operand32_e4m3");
  float v[32];
  bool bad = false;
  // element k of the operand: column 32g + k
#pragma unroll
  for (int c = 0; c < 4; ++c) {                      // four 8-element chunks
    const uint32_t h[4] = {qw[c].x, qw[c].y, qw[c].z, qw[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = h[e] & 0xFFFF, hi = h[e] >> 16;
      bad |= ((lo & 0x7F80) == 0x7F80) | ((hi & 0x7F80) == 0x7F80);
      v[8 * c + 2 * e] = bf16_bits_to_float(lo) * mult;
      v[8 * c + 2 * e + 1] = bf16_bits_to_float(hi) * mult;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k]));
  int x = amax > 0.0f ? floor_log2(amax) - Fmt<F>::emax : -127;
  x = x < -127 ? -127 : (x > 127 ? 127 : x);
  float y[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) y[k] = __builtin_ldexpf(v[k], -x);
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  Pack32<F, true>::run(y, w);
  if (bad) { for (int i = 0; i < 8; ++i) w[i] = 0; }
  sc = bad ? 255 : min(x + 127 + RAISE, 254);
  opv<F> o;
#pragma unroll
  for (int i = 0; i < Operand<F>::words; ++i) o[i] = (int)w[i];
  return o;
}

}  // namespace

}  // namespace fsa
