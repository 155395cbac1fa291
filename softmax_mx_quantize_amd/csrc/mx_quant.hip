// MX block quantiser for gfx950 (memory-bound).
//
// Block scale and element rounding follow the OCP Microscaling Formats v1.0
// rule for the MX operands the pages name (Fused-Softmax for efficient
// quantized attention, summary): X = clamp(floor(log2 amax) - emax, -127, 127),
// X = -127 for an all-zero block, elements x * 2^-X rounded to nearest-even
// and saturated, sign kept on zeros; a block holding NaN or Inf gets scale
// 0xFF and zero codes.  The power-of-two scaling is done with an exact
// ldexp; the rounding and packing use gfx950's scaled conversions with a
// unit scale.
//
// The fused attention path quantises Q multiplied by the softmax scale in
// binades (`mult`, one fp32 rounding per element); everything else uses 1.
//
// One thread owns one 32-element block.  Rows mode: the block runs along the
// contiguous axis and consecutive threads take consecutive blocks of a row
// (64-byte loads per thread, contiguous across the wave).  Columns mode: the
// block runs along the row axis and the output is transposed; consecutive
// threads take consecutive columns so each of the 32 loads is contiguous
// across the wave.
#include "fsa_device.h"
#include "fsa_internal.h"

namespace fsa {

template <int F, int MODE, bool VEC>
__global__ void __launch_bounds__(256) mx_quant_kernel(QuantArgs a) {
  constexpr int BITS = Fmt<F>::bits;
  constexpr int OUT_BYTES = 4 * BITS;   // 32 elements
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_out_rows = a.batch * a.out_rows;
  if (t >= n_out_rows * a.nb_out) return;
  int64_t o, b;
  if (MODE == 0) { o = t / a.nb_out; b = t - o * a.nb_out; }
  else           { o = t % n_out_rows; b = t / n_out_rows; }

  float v[32];
  bool bad = false;
  if (MODE == 0) {
    const int64_t bt = o / a.out_rows;
    const int64_t r = o - bt * a.out_rows;
    const int64_t c0 = b * 32;
    const bool row_ok = r < a.rows;
    const uint16_t* src = a.x + (bt * a.rows + r) * a.cols + c0;
    if (VEC && row_ok && c0 + 32 <= a.cols) {
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 q = s4[i];
        uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t lo = w[k] & 0xFFFF, hi = w[k] >> 16;
          bad |= ((lo & 0x7F80) == 0x7F80) | ((hi & 0x7F80) == 0x7F80);
          v[8 * i + 2 * k] = bf16_bits_to_float(lo) * a.mult;
          v[8 * i + 2 * k + 1] = bf16_bits_to_float(hi) * a.mult;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        uint32_t bits = 0;
        if (row_ok && c0 + j < a.cols) bits = src[j];
        bad |= (bits & 0x7F80) == 0x7F80;
        v[j] = bf16_bits_to_float(bits) * a.mult;
      }
    }
  } else {
    // o = (batch, column); the block covers rows [32b, 32b+32)
    const int64_t bt = o / a.cols;
    const int64_t c = o - bt * a.cols;
    const int64_t r0 = b * 32;
    const uint16_t* src = a.x + (bt * a.rows) * a.cols + c;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t bits = 0;
      if (r0 + j < a.rows) bits = src[(r0 + j) * a.cols];
      bad |= (bits & 0x7F80) == 0x7F80;
      v[j] = bf16_bits_to_float(bits) * a.mult;
    }
  }

  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  int X = amax > 0.0f ? floor_log2(amax) - Fmt<F>::emax : -127;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  float y[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = __builtin_ldexpf(v[j], -X);
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  Pack32<F, true>::run(y, w);
  uint8_t sbyte = (uint8_t)(X + 127);
  if (bad) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0;
    sbyte = 0xFF;
  }
  uint8_t* dst = a.codes + o * a.code_stride + b * OUT_BYTES;
  if (BITS == 8) {
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d4[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else if (BITS == 6) {
    uint2* d2 = reinterpret_cast<uint2*>(dst);
    d2[0] = make_uint2(w[0], w[1]);
    d2[1] = make_uint2(w[2], w[3]);
    d2[2] = make_uint2(w[4], w[5]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  int64_t so = o * a.scale_stride + b;
  if (a.scale_layout == SCALES_KEY_TILES) {
    // o = (batch, key row), b = block along D; rows per batch entry are a
    // whole number of 128-key tiles
    const int nb = (int)a.nb_out;
    const int64_t bt = o / a.out_rows;
    const int64_t row = o - bt * a.out_rows;
    const int rl = (int)(row & 127);
    const int r = BITS == 8 ? 4 * ((rl >> 4) & 3) + (rl & 3) : 4 * (rl >> 5) + (rl & 3);
    const int j = BITS == 8 ? ((rl >> 2) & 3) + 4 * (rl >> 6) : (rl >> 2) & 7;
    so = bt * a.out_rows * nb + (row >> 7) * 128 * nb + (r * nb + b) * 8 + j;
  } else if (a.scale_layout == SCALES_DIM_TILES) {
    // o = (batch, d), b = key block; blocks per row are a whole number of
    // 4-block tiles
    const int64_t bt = o / a.out_rows;
    const int d = (int)(o - bt * a.out_rows);
    const int ndt = (int)(a.out_rows / 16);
    so = bt * a.out_rows * a.nb_out + (b >> 2) * 4 * a.out_rows +
         ((d & 15) * 4 + (int)(b & 3)) * ndt + (d >> 4);
  }
  a.scales[so] = sbyte;
}

template <int F, int MODE>
static hipError_t launch_quant_fmt(const QuantArgs& a, hipStream_t stream) {
  const int64_t total = a.batch * a.out_rows * a.nb_out;
  const int64_t grid = (total + 255) / 256;
  const bool vec = MODE == 0 && (a.cols % 32 == 0) &&
                   ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL((mx_quant_kernel<F, MODE, true>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((mx_quant_kernel<F, MODE, false>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const QuantArgs& a, int fmt, int mode, hipStream_t stream) {
  if (mode == 0) {
    if (fmt == FMT_E4M3) return launch_quant_fmt<FMT_E4M3, 0>(a, stream);
    if (fmt == FMT_E2M3) return launch_quant_fmt<FMT_E2M3, 0>(a, stream);
    return launch_quant_fmt<FMT_E2M1, 0>(a, stream);
  }
  if (fmt == FMT_E4M3) return launch_quant_fmt<FMT_E4M3, 1>(a, stream);
  if (fmt == FMT_E2M3) return launch_quant_fmt<FMT_E2M3, 1>(a, stream);
  return launch_quant_fmt<FMT_E2M1, 1>(a, stream);
}

}  // namespace fsa
