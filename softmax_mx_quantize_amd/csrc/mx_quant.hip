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
// block runs along the row axis and the output is transposed; a workgroup
// stages a 128-row x 32-column tile in LDS with 16-byte loads first.
#include <type_traits>

#include "fsa_device.h"
#include "fsa_internal.h"

namespace fsa {

// The block's largest magnitude and whether it holds NaN or Inf, from the
// bf16 bit patterns alone: below the exponent field's top, magnitudes order
// as their low 15 bits do, and a NaN or Inf element has those bits at
// 0x7F80 or above.  Multiplying the largest magnitude by a.mult gives the
// largest |x * mult| exactly (rounding is monotone), so the values need no
// comparisons of their own.
struct BlockMax {
  uint32_t m = 0;
  __device__ __forceinline__ void add(uint32_t bits) { m = max(m, bits & 0x7FFFu); }
  __device__ __forceinline__ bool bad() const { return m >= 0x7F80u; }
  __device__ __forceinline__ float amax(float mult) const { return bf16_bits_to_float(m) * mult; }
};

// Quantise one block of 32 values (already multiplied by a.mult) whose
// largest magnitude is amax, and write its codes and scale byte: slab w,
// output row r, block b.
template <int F>
__device__ __forceinline__ void quantize_block(const QuantArgs& a, float (&v)[32], float amax, bool bad,
                                               int64_t w, int64_t r, int64_t b) {
  constexpr int BITS = Fmt<F>::bits;
  constexpr int OUT_BYTES = 4 * BITS;   // 32 elements
  int X = amax > 0.0f ? floor_log2(amax) - Fmt<F>::emax : -127;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  float y[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = __builtin_ldexpf(v[j], -X);
  uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  Pack32<F, true>::run(y, wd);
  uint8_t sbyte = (uint8_t)(X + 127);
  if (bad) {
#pragma unroll
    for (int i = 0; i < 8; ++i) wd[i] = 0;
    sbyte = 0xFF;
  }
  uint8_t* dst = a.codes + w * a.code_slab + r * (a.nb_out * OUT_BYTES) + b * OUT_BYTES;
  if (BITS == 8) {
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    d4[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  } else if (BITS == 6) {
    uint2* d2 = reinterpret_cast<uint2*>(dst);
    d2[0] = make_uint2(wd[0], wd[1]);
    d2[1] = make_uint2(wd[2], wd[3]);
    d2[2] = make_uint2(wd[4], wd[5]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  const int64_t nb = a.nb_out;
  int64_t so = (w * a.out_rows + r) * nb + b;
  if (a.scale_layout == SCALES_KEY_TILES) {
    // r = key row, b = block along D; rows per slab are a whole number of
    // 128-key tiles
    so = w * a.out_rows * nb + (r >> 7) * 128 * nb +
         key_tile_byte((int)(r & 127), (int)b, 32 * (int)nb, a.key8 ? 8 : BITS);
  } else if (a.scale_layout == SCALES_DIM_TILES) {
    // r = d, b = key block; blocks per row are a whole number of 4-block tiles
    so = w * a.out_rows * nb + (b >> 2) * 4 * a.out_rows + dim_tile_byte((int)r, (int)(b & 3), (int)a.out_rows);
  }
  a.scales[so] = sbyte;
}

__device__ __forceinline__ const uint16_t* slab_input(const QuantArgs& a, int64_t w) {
  const int64_t b = w / a.nh;
  return a.x + b * a.x_sb + (w - b * a.nh) * a.x_sh;
}

// Rows mode: blocks along the contiguous axis; one thread per block,
// consecutive threads take consecutive blocks of a row (64-byte loads per
// thread, contiguous across the wave).
template <int FSET, bool VEC>
__global__ void __launch_bounds__(256) mx_quant_rows_kernel(QuantArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_out_rows = a.batch * a.out_rows;
  if (t >= n_out_rows * a.nb_out) return;
  const int64_t o = t / a.nb_out;
  const int64_t b = t - o * a.nb_out;
  float v[32];
  BlockMax bm;
  const int64_t w = o / a.out_rows;
  const int64_t r = o - w * a.out_rows;
  const int64_t c0 = b * 32;
  const bool row_ok = r < a.rows;
  const uint16_t* src = slab_input(a, w) + r * a.x_sr + c0;
  if (VEC && row_ok && c0 + 32 <= a.cols) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 q = s4[i];
      uint32_t wq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lo = wq[k] & 0xFFFF, hi = wq[k] >> 16;
        bm.add(lo);
        bm.add(hi);
        v[8 * i + 2 * k] = bf16_bits_to_float(lo) * a.mult;
        v[8 * i + 2 * k + 1] = bf16_bits_to_float(hi) * a.mult;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t bits = 0;
      if (row_ok && c0 + j < a.cols) bits = src[j];
      bm.add(bits);
      v[j] = bf16_bits_to_float(bits) * a.mult;
    }
  }
  const bool bad = bm.bad();
  if (bad && a.nan_key) atomicMin(reinterpret_cast<unsigned long long*>(a.nan_key + w), (unsigned long long)r);
  const int f = (FSET & (FSET - 1)) ? a.fmt[w % a.nh] : 0;
  const float amax = bm.amax(a.mult);
  with_format<FSET>(f, [&](auto F) { quantize_block<decltype(F)::value>(a, v, amax, bad, w, r, b); });
}

// Columns mode: blocks run along the row axis and the output is transposed.
// A workgroup of 128 threads stages a tile of 128 input rows x 32 columns in
// LDS with 16-byte loads (a row segment of 64 bytes per input row), then
// thread (column c = t % 32, block kb = t / 32) quantises the 32 rows of
// block kb in its column.  Row tiles run fastest in the grid: with 128 row
// tiles per slab (or any multiple of 8), the workgroup that reads the other
// half of a row's 128-byte lines runs on the same XCD and finds them in its
// L2.  Measured slower: column blocks fastest (the halves spread over XCDs,
// +25 %), and 128 x 64 tiles of whole lines on 256 threads (+4 %).
constexpr int QC_ROWS = 128, QC_COLS = 32;
template <int FSET, bool VEC>
__global__ void __launch_bounds__(128) mx_quant_cols_kernel(QuantArgs a) {
  __shared__ __align__(16) uint16_t tile[QC_ROWS][QC_COLS];
  const int t = threadIdx.x;
  const int64_t w = a.batch0 + blockIdx.z;
  if (a.nan_init && blockIdx.x == 0 && blockIdx.y == 0 && t == 0) a.nan_key[w] = ~0ull;
  const int64_t col0 = (int64_t)blockIdx.y * QC_COLS;
  const int64_t row0 = (int64_t)blockIdx.x * QC_ROWS;
  const uint16_t* src = slab_input(a, w);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + 128 * i;               // 16-byte chunk: row c/4, part c%4
    const int row = c >> 2, part = c & 3;
    const int64_t gr = row0 + row, gc = col0 + part * 8;
    uint4 q = make_uint4(0, 0, 0, 0);
    if (VEC) {
      if (gr < a.rows && gc + 8 <= a.cols)
        q = *reinterpret_cast<const uint4*>(src + gr * a.x_sr + gc);
    } else if (gr < a.rows) {
      uint32_t hq[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hq[e] = gc + e < a.cols ? src[gr * a.x_sr + gc + e] : 0u;
      q = make_uint4(hq[0] | (hq[1] << 16), hq[2] | (hq[3] << 16), hq[4] | (hq[5] << 16), hq[6] | (hq[7] << 16));
    }
    *reinterpret_cast<uint4*>(&tile[row][part * 8]) = q;
  }
  __syncthreads();
  const int cc = t & 31, kb = t >> 5;
  const int64_t col = col0 + cc;
  const int64_t b = (int64_t)blockIdx.x * (QC_ROWS / 32) + kb;
  if (col >= a.cols || b >= a.nb_out) return;
  float v[32];
  BlockMax bm;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t bits = tile[32 * kb + j][cc];
    bm.add(bits);
    v[j] = bf16_bits_to_float(bits) * a.mult;
  }
  const bool bad = bm.bad();
  const float amax = bm.amax(a.mult);
  const int f = (FSET & (FSET - 1)) ? a.fmt[w % a.nh] : 0;
  with_format<FSET>(f, [&](auto F) { quantize_block<decltype(F)::value>(a, v, amax, bad, w, col, b); });
}

template <int FSET>
static hipError_t launch_quant_set(const QuantArgs& a, int mode, hipStream_t stream) {
  // 16-byte loads need every row start 16-byte aligned
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 && a.x_sr % 8 == 0 &&
                       a.x_sh % 8 == 0 && a.x_sb % 8 == 0;
  if (mode == 0) {
    const int64_t total = a.batch * a.out_rows * a.nb_out;
    const int64_t grid = (total + 255) / 256;
    if (a.cols % 32 == 0 && aligned)
      hipLaunchKernelGGL((mx_quant_rows_kernel<FSET, true>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((mx_quant_rows_kernel<FSET, false>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  } else {
    // slabs go in grid.z, in launches of at most 65535
    for (int64_t b0 = 0; b0 < a.batch; b0 += 65535) {
      QuantArgs c = a;
      c.batch0 = b0;
      const int64_t nb = a.batch - b0 < 65535 ? a.batch - b0 : 65535;
      const dim3 grid((unsigned)((a.nb_out + QC_ROWS / 32 - 1) / (QC_ROWS / 32)),
                      (unsigned)((a.cols + QC_COLS - 1) / QC_COLS), (unsigned)nb);
      if (a.cols % 8 == 0 && aligned)
        hipLaunchKernelGGL((mx_quant_cols_kernel<FSET, true>), grid, dim3(128), 0, stream, c);
      else
        hipLaunchKernelGGL((mx_quant_cols_kernel<FSET, false>), grid, dim3(128), 0, stream, c);
    }
  }
  return hipGetLastError();
}

hipError_t launch_mx_quant(const QuantArgs& a, int fset, int mode, hipStream_t stream) {
  switch (fset) {
    case 1 << FMT_E4M3: return launch_quant_set<1 << FMT_E4M3>(a, mode, stream);
    case 1 << FMT_E2M3: return launch_quant_set<1 << FMT_E2M3>(a, mode, stream);
    case 1 << FMT_E2M1: return launch_quant_set<1 << FMT_E2M1>(a, mode, stream);
    default: return launch_quant_set<7>(a, mode, stream);
  }
}

}  // namespace fsa
