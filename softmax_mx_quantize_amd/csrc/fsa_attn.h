// The fused-softmax attention kernel: its body per element format and P~
// variant, the kernel over a set of formats, and its launch templates.
// Included by the translation units that instantiate them.
#pragma once

// Fused-Softmax attention forward for MXFP8 (E4M3), MXFP6 (E2M3) and MXFP4
// (E2M1) operands on the 32x32x64 scaled MFMA of gfx950.
//
// The steps (frozen max, score product with the exponential's linear part
// folded in, per-32-key bit-pattern exponential and MX quantisation of P,
// P V and row sums on the matrix cores, power-of-two re-basing of rows above
// their guess, normalisation) are listed in fsa_common.h, with the citations
// of the pages.  The products use the 32x32x64 form: it does twice the work
// of the 16x16x128 one per instruction for about the same occupancy of the
// wave's issue port, and it lets a lane hold the 32 keys it supplies to the
// P V product.
//
// Register layout (32x32x64 scaled MFMA, lane (h, n) = 32 h + n):
//   * A row n / B column n; FP6/FP4 operands hold K elements [32h, 32h+32)
//     with the lane's own E8M0 scale: one lane = one MX block; FP8 operands
//     hold [16h, +16) in bytes 0-15 and [32+16h, +16) in bytes 16-31, and
//     the scale of K block c (elements [32c, +32)) is lane half c's;
//   * output register i of lane (h, n) is row 8 (i/4) + 4 h + i%4, column n.
// The score tile is computed transposed (keys as rows, the wave's 32 queries
// as columns) over 64-key chunks: block b in {0, 1} of chunk u takes as its A
// row rho = 8 j + 4 x + k the key 32 x + 16 b + 4 j + k of the chunk (FP8:
// 32 b + 16 x + 4 j + k), so that register i of lane (h, n) in block b is key
// 32 h + 16 b + i (FP8: 32 b + 16 h + i).  A lane then holds exactly the 32
// keys of one query that it supplies as the B operand of O^T += V^T P~^T
// over that chunk: for FP6/FP4 one whole MX block of P, whose maximum and
// scale need no lane exchange; for FP8 half of each of the chunk's blocks.
//
// Row sums l += 1 P~^T.  FP6/FP4: one 16x16x128 product per chunk with an
// FP4 ones operand: in that product lane 16 g + c supplies K elements
// [32g, 32g+32) of column c, i.e. chunk keys [32 (g/2), +32) of query
// 16 (g%2) + c, so ones in the A rows 0-7 for even g and rows 8-15 for odd g
// give, in output rows 0-7, the sum of query c and in rows 8-15 that of query
// 16 + c.  FP8: that product's B operand would share one scale between the
// half blocks of two queries, so the sum takes a 32x32x64 product with an
// all-ones FP4 operand instead (every output row is the column's sum).
#include "fsa_common.h"

namespace fsa {

__device__ v16f mfma32_v6(v6i a, v6i b, v16f c, int cbsz, int blgp, int opsel_a, int sa,
                          int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v6i32.v6i32");
__device__ v16f mfma32_v4(v4i a, v4i b, v16f c, int cbsz, int blgp, int opsel_a, int sa,
                          int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");
// FP4 / FP6 A operand with an FP8 B operand (row sums of FP8
// probabilities; V^T products of E4M3 P~ over FP6/FP4 operands).
__device__ v16f mfma32_v4_v8(v4i a, v8i b, v16f c, int cbsz, int blgp, int opsel_a, int sa,
                             int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v8i32");
__device__ v16f mfma32_v6_v8(v6i a, v8i b, v16f c, int cbsz, int blgp, int opsel_a, int sa,
                             int opsel_b, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v6i32.v8i32");

namespace {

template <int F, int OA>
__device__ __forceinline__ v16f mma32(const opv<F>& a, const opv<F>& b, const v16f& c, int sa,
                                      int sb) {
  if constexpr (Fmt<F>::bits == 8)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma, OA,
                                                           sa, 0, sb);
  else if constexpr (Fmt<F>::bits == 6)
    return mfma32_v6(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma, OA, sa, 0, sb);
  else
    return mfma32_v4(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma, OA, sa, 0, sb);
}
// O^T += V^T P~^T with V^T in format F (A) and P~ in format P (B): the same
// format, E2M3 V^T with E3M2 P~ (same width, two element formats), or
// FP6/FP4 V^T with FP8 P~ (mixed widths).
template <int F, int P, int OA>
__device__ __forceinline__ v16f mma32_pv(const opv<F>& a, const opv<P>& b, const v16f& c, int sa,
                                         int sb) {
  if constexpr (F == P) return mma32<F, OA>(a, b, c, sa, sb);
  else if constexpr (Fmt<F>::bits == 6 && Fmt<P>::bits == 6)
    return mfma32_v6(a, b, c, Fmt<F>::mfma, Fmt<P>::mfma, OA, sa, 0, sb);
  else if constexpr (Fmt<F>::bits == 6)
    return mfma32_v6_v8(a, b, c, Fmt<F>::mfma, Fmt<P>::mfma, OA, sa, 0, sb);
  else
    return mfma32_v4_v8(a, b, c, Fmt<F>::mfma, Fmt<P>::mfma, OA, sa, 0, sb);
}
template <int F, int P>
__device__ __forceinline__ v16f mma32_pv_sel(const opv<F>& a, const opv<P>& b, const v16f& c, int sa,
                                             int byte, int sb) {
  switch (byte & 3) {
    case 0: return mma32_pv<F, P, 0>(a, b, c, sa, sb);
    case 1: return mma32_pv<F, P, 1>(a, b, c, sa, sb);
    case 2: return mma32_pv<F, P, 2>(a, b, c, sa, sb);
    default: return mma32_pv<F, P, 3>(a, b, c, sa, sb);
  }
}

// A's scale byte chosen by a value that is a constant after unrolling.
template <int F>
__device__ __forceinline__ v16f mma32_sel(const opv<F>& a, const opv<F>& b, const v16f& c, int sa,
                                          int byte, int sb) {
  switch (byte & 3) {
    case 0: return mma32<F, 0>(a, b, c, sa, sb);
    case 1: return mma32<F, 1>(a, b, c, sa, sb);
    case 2: return mma32<F, 2>(a, b, c, sa, sb);
    default: return mma32<F, 3>(a, b, c, sa, sb);
  }
}

// XOR swizzles of the 16-byte chunk of a 128-byte LDS row.  The LDS has 64
// banks of 4 bytes (two rows per bank line, the row's parity picks the half)
// and serves a 16-byte read 16 lanes at a time, so the 16 rows those lanes
// read need distinct chunks within each parity (the bank-conflict counter
// confirms it).  Score product: lanes n = 8j + 4x + k of one 16-lane group
// read key rows 32x + 16b + 4j + k (FP6/FP4) or 32b + 16x + 4j + k (FP8)
// (+64u): rows differing in bits 0, 1, 2 and 5 (FP8: 4).  P V product:
// lanes n read rows n (+32 db): bits 0-3.  FP6's 8-byte second piece is
// read 32 lanes at a time; its half of the chunk follows row bit 3 (K^) or 4
// (V^T), the fifth bit those 32 rows differ in.
template <int BITS>
__device__ __forceinline__ int swz_k32(int row) {
  return ((row >> 1) & 3) | (((row >> (BITS == 8 ? 4 : 5)) & 1) << 2);
}
__device__ __forceinline__ int swz_v32(int row) { return (row >> 1) & 7; }

// Columns of the pieces of the lane's FP8 Q' operand for 64-wide D chunk c:
// elements [64c + 16h, +16) and [64c + 32 + 16h, +16).
__device__ __forceinline__ void q_cols32(int c, int hh, int (&col)[4]) {
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) col[ch] = 64 * c + 16 * hh + (ch < 2 ? 8 * ch : 32 + 8 * (ch - 2));
}

// The lane's Q' operand for 64-wide D chunk c of the FP8 score product,
// from the bf16 words of q_words over q_cols32(c, hh): half of D block 2c
// and half of block 2c+1; the other halves are in the lane 32 apart.  Same
// rule as the quantiser (OCP floor scale, RNE, saturation, NaN/Inf blocks
// get scale 0xFF and zero codes), Q' = fp32(q * mult), 2^23 raised onto the
// E8M0 byte.  `sc` is the byte of block 2c + h, which this lane supplies.
template <int RAISE>
__device__ __forceinline__ v8i q_operand32_e4m3(const uint4 (&qw)[4], float mult, int hh, int& sc) {
  float v[32];
  bool bad_lo = false, bad_hi = false;
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    const uint32_t hw[4] = {qw[ch].x, qw[ch].y, qw[ch].z, qw[ch].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = hw[e] & 0xFFFF, hi = hw[e] >> 16;
      const bool nan_inf = ((lo & 0x7F80) == 0x7F80) | ((hi & 0x7F80) == 0x7F80);
      if (ch < 2) bad_lo |= nan_inf; else bad_hi |= nan_inf;
      v[8 * ch + 2 * e] = bf16_bits_to_float(lo) * mult;
      v[8 * ch + 2 * e + 1] = bf16_bits_to_float(hi) * mult;
    }
  }
  float a_lo = 0.0f, a_hi = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    a_lo = __builtin_fmaxf(a_lo, __builtin_fabsf(v[k]));
    a_hi = __builtin_fmaxf(a_hi, __builtin_fabsf(v[16 + k]));
  }
  a_lo = __builtin_fmaxf(a_lo, __shfl_xor(a_lo, 32));
  a_hi = __builtin_fmaxf(a_hi, __shfl_xor(a_hi, 32));
  bad_lo |= __shfl_xor((int)bad_lo, 32) != 0;
  bad_hi |= __shfl_xor((int)bad_hi, 32) != 0;
  auto scale_exp = [](float amax) {
    int X = amax > 0.0f ? floor_log2(amax) - Fmt<FMT_E4M3>::emax : -127;
    return X < -127 ? -127 : (X > 127 ? 127 : X);
  };
  const int x_lo = scale_exp(a_lo), x_hi = scale_exp(a_hi);
  float y[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) y[k] = __builtin_ldexpf(v[k], -(k < 16 ? x_lo : x_hi));
  uint32_t w[8];
  Pack32<FMT_E4M3, true>::run(y, w);
  if (bad_lo) { for (int i = 0; i < 4; ++i) w[i] = 0; }
  if (bad_hi) { for (int i = 4; i < 8; ++i) w[i] = 0; }
  auto raised = [](int x, bool bad) { return bad ? 255 : min(x + 127 + RAISE, 254); };
  sc = hh ? raised(x_hi, bad_hi) : raised(x_lo, bad_lo);
  v8i o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (int)w[i];
  return o;
}

}  // namespace

// REBASE: the fallback pass of a call.  A workgroup does nothing unless
// the first pass stamped the call's flag and left one of its rows more than
// EXT binades above its frozen max; it then sweeps again from the reference
// raised by each row's offset kappa (whole binades, so no shift is clamped)
// and overwrites the rows the first pass left beyond EXT.  The first pass
// records kappa exactly below KSAT; only a workgroup with a row at KSAT or
// beyond first measures its rows' offsets from the fp32 scores in a
// scores-only sweep.
//
// One workgroup's work: query tile q_wg of head h of batch entry b, whose
// quantised K^ / V^T are slab wi of the workspace, in element format F.
// The LDS stages are the kernel's (their size depends on D only).
//
// F is the element format of Q'^, K^ and V^; P that of P~ (F, or E4M3 over
// FP6/FP4 operands); PM the P~ variant (PM_* in fsa_common.h).  The key
// order of the score rows, the K^ scale layout and the epilogue follow P.
template <int F, int P, int PM, int D, bool CAUSAL, bool REBASE>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const int b, const int h,
                                          const int64_t wi, const int q_wg, uint8_t* kl0,
                                          uint8_t* kl1, uint8_t* vl0, uint8_t* vl1) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource types exist only in the device pass
  constexpr int NWAVES = 4;
  constexpr int BITS = Fmt<F>::bits;         // operand codes
  constexpr int PBITS = Fmt<P>::bits;        // P~ codes
  constexpr bool KEY8 = PBITS == 8;          // FP8 key order of the score rows
  constexpr int KOB = KEY8 ? 8 : 4;          // key-order argument of the layouts
  static_assert(P == F || (P == FMT_E4M3 && PM == PM_BLOCK) ||
                    (P == FMT_E3M2 && F == FMT_E2M3 && PM == PM_BLOCK),
                "E4M3 P~ over FP6/FP4 operands, E3M2 P~ over E2M3 operands");
  static_assert(PM != PM_ROW || (F == FMT_E4M3 && P == FMT_E4M3), "one scale per row: E4M3");
  static_assert(PM != PM_EFQ || (F == FMT_E2M1 && P == FMT_E2M1), "affine codes: E2M1");
  // Exact exponential: the score product yields t + REF in binades (no 2^23
  // on Q's scale) and the vector unit's exp2 forms 2^(t + REF); otherwise the
  // product yields the bit pattern's exponent field directly.
  constexpr bool EXPX = PM == PM_EXP;
  constexpr int QRAISE = EXPX ? 0 : 23;
  constexpr float TO_Y = EXPX ? 8388608.0f : 1.0f;  // accumulator value -> 2^23 units

  static_assert(D == 64 || D == 128, "D is 64 or 128");
  constexpr int MB = Fmt<P>::mbits;
  // placement binade of P~ blocks (E4M3: one below the top, whose largest
  // code is NaN and whose values clip at 448)
  constexpr int PL = P == FMT_E4M3 ? Fmt<P>::emax - 1 : Fmt<P>::emax;
  constexpr int CAP = 127 - PL;
  constexpr int RB = D * BITS / 8;           // bytes per K^ row (global)
  constexpr int RS = 128;                    // bytes per K^ / V^T row (LDS)
  constexpr int VRB = KT * BITS / 8;         // bytes per V^T row of one tile (global)
  constexpr int ND = D / 64;                 // 64-wide D chunks of the score product
  constexpr int NDB = D / 32;                // 32-row blocks of O^T; MX blocks per K^ row
  constexpr int QW = NWAVES * 32;            // queries per workgroup
  // Operand fetches of a chunk's products: all of its K^ (KBATCH) or V^T
  // (VBATCH) fragments are read from LDS before its first product instead
  // of one product ahead.  Measured per format (Video-DiT shape): batching
  // the V^T reads gains ~1 % for FP8 and the K^ reads cost it ~1 %; K^ alone
  // gains ~1 % for FP6; both gain ~1.5 % for FP4.
  constexpr bool KBATCH = BITS != 8;
  constexpr bool VBATCH = BITS != 6;
  constexpr int K_BYTES = KT * RS;
  constexpr int V_BYTES = D * RS;
  constexpr int KS_BYTES = KT * NDB;
  constexpr int VS_BYTES = 4 * D;
  constexpr int KSTAGE = K_BYTES + KS_BYTES;
  constexpr int VSTAGE = V_BYTES + VS_BYTES;
  constexpr int NBK = KS_BYTES / 64;         // K^ scale bytes per lane and tile
  constexpr int NBV = VS_BYTES / 64;         // V^T scale bytes per lane and tile
  constexpr int XLO = 127 + REF - CAP, XHI = 127 + REF + EXT;
  // LDS rows.  FP8 and FP4: logical chunk c is bytes [16c, 16c+16) of the
  // row.  FP6: each 24-byte block b takes two chunks, 2b (its bytes 0-15)
  // and 2b+1 (bytes 16-23 in one half), so that a lane's operand is one
  // 16-byte and one 8-byte read into consecutive registers.
  constexpr int NPC = BITS == 4 ? 1 : 2;     // LDS reads per operand
  // Score rows: block b of a chunk steps KB rows, the A row's x bit KX rows.
  constexpr int KB = KEY8 ? 32 : 16, KX = KEY8 ? 16 : 32;

  // Two-stage rings (two workgroups share a CU); one LDS object per stage,
  // always addressed through a compile-time stage index so that the
  // compiler sees that reads of one stage never alias the DMA into the other.
  static_assert(KSTAGE == attn_kstage_bytes(D) && VSTAGE == attn_vstage_bytes(D), "LDS stages");
  auto kstage = [&](auto st_tag) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(st_tag)::value == 0) return kl0; else return kl1;
  };
  auto vstage = [&](auto st_tag) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(st_tag)::value == 0) return vl0; else return vl1;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;                  // lane half
  const int n = lane & 31;                   // query column / A row of the products

  const int64_t bh = (int64_t)b * a.H + h;
  const int S = a.S;
  const int q_wave = q_wg + wave * 32;
  const int q = q_wave + n;                  // this lane's query

  // slabs of the widest format in the launch; this head's rows are packed
  // in its own format at their start
  const uint8_t* kc = a.kc + wi * a.kc_slab;
  const uint8_t* ks = a.ks + wi * (int64_t)a.sk_alloc * NDB;
  const int64_t v_row = (int64_t)a.sk_alloc * BITS / 8;
  const uint8_t* vc = a.vc + wi * a.vc_slab;
  const int vs_row = a.sk_alloc / 32;
  const uint8_t* vs = a.vs + wi * (int64_t)D * vs_row;

  int n_tiles = (S + KT - 1) / KT;
  if (CAUSAL) {
    const int last_q = q_wg + QW - 1 < S - 1 ? q_wg + QW - 1 : S - 1;
    n_tiles = min(n_tiles, last_q / KT + 1);
  }

  // ---- direct global -> LDS copies (each instruction: 8 LDS rows of 8
  // chunks per wave; lane i fills physical chunk i%8 of row i/8 with the
  // logical chunk the swizzle maps there; chunks past a row's data re-read
  // its chunk 0).  Row R = 8 (wave + 4k) + i/8: its bits 1-2 come from i/8,
  // bits 3-4 from the wave and bit 5 from k, so a lane needs one K^ offset
  // for even and one for odd k, and one V^T offset.  The tile and row
  // offsets go in the scalar operand.
  constexpr int NK_DMA = KT * 8 / 64 / NWAVES;
  constexpr int NV_DMA = D * 8 / 64 / NWAVES;
  constexpr int NKS = KS_BYTES / 256;
  constexpr int NVS = VS_BYTES / 256;
  static_assert(NKS >= 1 && NKS <= NWAVES && NVS >= 1 && NVS <= NWAVES, "scale loads");
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kc, (short)0, a.sk_alloc * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vc, (short)0, (int)(D * v_row), 0x00020000);
  const __amdgpu_buffer_rsrc_t ks_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)ks, (short)0, a.sk_alloc * NDB, 0x00020000);
  const __amdgpu_buffer_rsrc_t vs_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vs, (short)0, D * vs_row, 0x00020000);
  // Global byte of logical chunk c within a row of `nblk` MX blocks
  // (chunks past the row's data re-read its first bytes).
  // FP6: `hs` = 1 puts block bytes 16-23 in the upper half of their chunk
  // (rows with bit 3 set for K^, bit 4 for V^T), so that the 32 lanes reading
  // those 8-byte pieces together spread over both halves of the bank line.
  auto chunk_src = [](int c, int nblk, int hs) __attribute__((always_inline)) {
    if constexpr (BITS == 6) return (c >> 1) < nblk ? 24 * (c >> 1) + (c & 1) * (16 - 8 * hs) : 0;
    else return c < nblk * BITS / 4 ? 16 * c : 0;
  };
  auto k_hs = [](int row) __attribute__((always_inline)) { return (row >> 3) & 1; };
  auto v_hs = [](int row) __attribute__((always_inline)) { return (row >> 4) & 1; };
  int koff_e, koff_o, voff;
  {
    const int r_e = 8 * wave + (lane >> 3), r_o = r_e + 8 * NWAVES;   // rows of even / odd k
    koff_e = (lane >> 3) * RB + chunk_src((lane & 7) ^ swz_k32<KOB>(r_e), NDB, k_hs(r_e));
    koff_o = (lane >> 3) * RB + chunk_src((lane & 7) ^ swz_k32<KOB>(r_o), NDB, k_hs(r_o));
    const int c = (lane & 7) ^ swz_v32(r_e);
    voff = (lane >> 3) * (int)v_row + chunk_src(c, 4, v_hs(r_e));
  }
  const int s_voff = lane * 4;
  auto issue_k = [&](int t, uint8_t* base) __attribute__((always_inline)) {
    const uint32_t lb = lds_addr(base);
    const int ks_soff = wave < NKS ? wave * 256 : 0;
#pragma unroll
    for (int k = 0; k < NK_DMA; ++k)
      dma_lds16(k_rsrc, lb + (wave + NWAVES * k) * 1024, (k & 1) ? koff_o : koff_e,
                t * KT * RB + (wave + NWAVES * k) * 8 * RB);
    dma_lds4(ks_rsrc, lb + K_BYTES + ks_soff, s_voff, t * KS_BYTES + ks_soff);
  };
  auto issue_v = [&](int t, uint8_t* base) __attribute__((always_inline)) {
    const uint32_t lb = lds_addr(base);
    const int vs_soff = wave < NVS ? wave * 256 : 0;
#pragma unroll
    for (int k = 0; k < NV_DMA; ++k)
      dma_lds16(v_rsrc, lb + (wave + NWAVES * k) * 1024, voff,
                t * VRB + (wave + NWAVES * k) * 8 * (int)v_row);
    dma_lds4(vs_rsrc, lb + V_BYTES + vs_soff, s_voff, t * VS_BYTES + vs_soff);
  };

  // first pass's offset of this lane's row (REBASE)
  [[maybe_unused]] int kap_in = 0;
  if constexpr (REBASE) {
    if (*a.fb_flag != a.call_id) return;                    // the same for every workgroup
    kap_in = q < S ? a.row_kappa[(bh - a.row_bh0) * S + q] : 0;
    if (!__syncthreads_or(kap_in > EXT)) return;            // the same for the whole workgroup
  }

  if (n_tiles > 0) {
    issue_k(0, kl0);
    issue_v(0, vl0);
  }

  // ---- Q' operands (B of the score product), one per 64-wide D chunk c:
  // lane (h, n) holds D block 2c + h of query n, quantised here from the
  // bf16 row with 2^23 on its E8M0 scale
  opv<F> qf[ND];
  int qsc[ND];
  {
    // every chunk's words first (one wait for all of them), then the codes;
    // a padding row reads the last row and zeroes it
    const uint16_t* qrow = a.q + b * a.q_sb + h * a.q_sh + (int64_t)(q < S ? q : S - 1) * a.q_ss;
    uint4 qw[ND][4];
#pragma unroll
    for (int c = 0; c < ND; ++c) {
      int col[4];
      if constexpr (BITS == 8) q_cols32(c, hh, col);
      else q_cols(2 * c + hh, col);
      q_words(qrow, q < S, col, qw[c]);
    }
    // (left to itself the FP8 schedule issues the second chunk's loads only
    // after the first chunk's codes)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < ND; ++c) {
      if constexpr (BITS == 8) qf[c] = q_operand32_e4m3<QRAISE>(qw[c], a.qmul, hh, qsc[c]);
      else qf[c] = q_operand<F, QRAISE>(qw[c], a.qmul, qsc[c]);
    }
  }

  // ---- lane-constant LDS offsets.  Score product, chunk u, block b, D chunk
  // c: A row n reads key row 64u + 16b + krow0 at logical byte
  // (64c + 32h) * BITS/8 (+8 per FP6 piece); the swizzle of those rows does
  // not depend on u or b.  P V product, chunk u, block db: A row n reads
  // V^T row 32 db + n at logical byte (64u + 32h) * BITS/8.
  const int krow0 = KX * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  const int ksw = swz_k32<KOB>(krow0);
  const int vsw = swz_v32(n);
  // logical chunk of piece p of the lane's part of 64-element chunk m of a
  // row (FP8: elements [64m + 16h, +16) and [64m + 32 + 16h, +16); FP6/FP4:
  // MX block 2m + h)
  auto piece_chunk = [&](int m, int p) __attribute__((always_inline)) {
    if constexpr (BITS == 8) return 4 * m + 2 * p + hh;
    else if constexpr (BITS == 6) return 2 * (2 * m + hh) + p;
    else return 2 * m + hh;
  };
  int k_off[ND][NPC], v_off[2][NPC];
#pragma unroll
  for (int c = 0; c < ND; ++c)
#pragma unroll
    for (int p = 0; p < NPC; ++p)
      k_off[c][p] = krow0 * RS + 16 * (piece_chunk(c, p) ^ ksw) + (BITS == 6 && p == 1 ? 8 * k_hs(krow0) : 0);
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int p = 0; p < NPC; ++p)
      v_off[u][p] = n * RS + 16 * (piece_chunk(u, p) ^ vsw) + (BITS == 6 && p == 1 ? 8 * v_hs(n) : 0);
  auto frag = [&](const uint8_t* base, const int* off, int imm) __attribute__((always_inline)) -> opv<F> {
    opv<F> o;
    if constexpr (BITS == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + off[0] + imm);
      const uint4 w = *reinterpret_cast<const uint4*>(base + off[1] + imm);
      o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; o[4] = w.x; o[5] = w.y; o[6] = w.z; o[7] = w.w;
    } else if constexpr (BITS == 6) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + off[0] + imm);
      // the 8-byte piece's address is made opaque: left visible, the
      // compiler pairs the pieces of blocks 16 or 32 rows apart into one
      // ds_read2st64_b64, whose two addresses hit the same banks (measured:
      // a third of the LDS cycles in bank conflicts, 3 % slower)
      int a1 = off[1] + imm;
      asm volatile("" : "+v"(a1));
      const uint2 w = *reinterpret_cast<const uint2*>(base + a1);
      o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; o[4] = w.x; o[5] = w.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(base + off[0] + imm);
      o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    return o;
  };
  auto kfrag = [&](const uint8_t* base, int u, int bb, int c) __attribute__((always_inline)) {
    return frag(base, k_off[c], (64 * u + KB * bb) * RS);
  };
  auto vfrag = [&](const uint8_t* base, int u, int db) __attribute__((always_inline)) {
    return frag(base, v_off[u], 32 * db * RS);
  };
  // Scale bytes of the tile (tile-ordered: lane * NB): dword, then byte.
  auto k_scales = [&](const uint8_t* base) __attribute__((always_inline)) -> uint2 {
    if constexpr (NBK == 8) return *reinterpret_cast<const uint2*>(base + K_BYTES + lane * 8);
    else return make_uint2(*reinterpret_cast<const uint32_t*>(base + K_BYTES + lane * 4), 0u);
  };
  auto v_scales = [&](const uint8_t* base) __attribute__((always_inline)) -> uint2 {
    if constexpr (NBV == 8) return *reinterpret_cast<const uint2*>(base + V_BYTES + lane * 8);
    else return make_uint2(*reinterpret_cast<const uint32_t*>(base + V_BYTES + lane * 4), 0u);
  };
  auto pick = [](const uint2& s, int byte) __attribute__((always_inline)) {
    return (int)(byte < 4 ? s.x : s.y);
  };

  const v16f zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Key (within the tile) of output register i of block b of chunk u in
  // this lane: 64u + 32h + 16b + i (FP6/FP4), 64u + 32b + 16h + i (FP8).
  auto ckey = [&](int u, int bb, int i) __attribute__((always_inline)) {
    return 64 * u + (KEY8 ? 32 * bb + 16 * hh : 32 * hh + 16 * bb) + i;
  };

  // ---- frozen max from the first tile (keys [0, 128)); register i of lane
  // (h, n) in block b of chunk u is key 64u + 32h + 16b + i
  float mg;
  wait_dma();
  __syncthreads();
  if (n_tiles > 1) { issue_k(1, kl1); issue_v(1, vl1); }
  if constexpr (REBASE) {
    mg = q < S ? a.row_mguess[(bh - a.row_bh0) * S + q] : 0.0f;
  } else {
    const uint2 ksc = k_scales(kl0);
    v16f s0[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int c = 0; c < ND; ++c) {
          const int byte = u * 2 * ND + bb * ND + c;
          s0[u][bb] = mma32_sel<F>(kfrag(kl0, u, bb, c), qf[c], c == 0 ? zero16 : s0[u][bb],
                                   pick(ksc, byte), byte, qsc[c]);
        }
    float sum = 0.f, mx = -INFINITY;
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = ckey(u, bb, i);
          const bool vis = key < S && (!CAUSAL || key <= q);
          const float x = s0[u][bb][i];
          sum += vis ? x : 0.f;
          mx = vis ? __builtin_fmaxf(mx, x) : mx;
          cnt += vis ? 1 : 0;
        }
    sum += __shfl_xor(sum, 32);
    cnt += __shfl_xor(cnt, 32);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float mean = sum / (float)(cnt > 0 ? cnt : 1);
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = ckey(u, bb, i);
          const bool vis = key < S && (!CAUSAL || key <= q);
          const float dlt = s0[u][bb][i] - mean;
          ss += vis ? dlt * dlt : 0.f;
        }
    ss += __shfl_xor(ss, 32);
    const float sd = __builtin_sqrtf(ss / (float)(cnt > 0 ? cnt : 1));
    const int nvis = CAUSAL ? (q + 1 < S ? q + 1 : S) : S;
    const float z = __builtin_sqrtf(2.0f * __builtin_logf((float)nvis)) + 1.0f;
    // statistics of 2^23 s (or s), back to binades (exact power-of-two
    // scaling); the guess leads the window max by at most GUESS_CAP binades,
    // so that no row lies beyond the block shifts' reach below it
    constexpr float CAPU = (float)GUESS_CAP * (EXPX ? 1.0f : 8388608.0f);
    mg = __builtin_fminf(__builtin_fmaxf(mx, mean + z * sd), mx + CAPU) * (EXPX ? 1.0f : 0x1p-23f) +
         a.bias;
    // stored now, so that it need not stay live across the sweep
    if (q < S && hh == 0) a.row_mguess[(bh - a.row_bh0) * S + q] = mg;
  }

  // ---- main sweep (no online max, no rescaling; a block above the guess
  // takes a larger E8M0 scale, rows beyond EXT binades go to the fallback)
  v16f O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = zero16;
  // Row sums.  FP6/FP4 P~: a 16x16x128 product (see the head of this file).
  // FP8 P~: a 32x32x64 product with an all-ones FP4 A operand (every output
  // row is the sum of column n), because the FP8 16x16x128 B operand shares
  // one scale between the half blocks of two queries.  (With one scale per
  // row that sharing would be harmless, but that product's sums did not
  // match the P V products' on rows full of subnormal codes: V = 1 no longer
  // gave exactly 1, so the row sums stay on the product shape of P V.)
  constexpr bool L32 = PBITS == 8;
  using LAcc = std::conditional_t<L32, v16f, v4f>;
  LAcc L;
#pragma unroll
  for (int i = 0; i < (L32 ? 16 : 4); ++i) L[i] = 0.f;
  int kmax = -1000000;
  uint32_t over = 0;                         // one scale per row: overflow bits
  // accumulator start: fp32(2^23 (127 + R) - 2^23 m~), one rounding (exact
  // exponential: R - m~ in binades)
  float c0 = EXPX ? (float)REF - mg : __builtin_fmaf(-8388608.0f, mg, 8388608.0f * (127 + REF));
  v16f minit;
#pragma unroll
  for (int i = 0; i < 16; ++i) minit[i] = c0;
  // FP4 ones of the row-sum product: all ones for the 32x32 one; for FP6/FP4
  // P~ ones in A rows 0-7 for even lane groups and rows 8-15 for odd ones.
  v4i ones;
  {
    const int on = L32 || ((lane >> 4) & 1) == ((lane & 15) >> 3) ? 0x22222222 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) ones[i] = on;
  }

  v16f acc[2][2];
  opv<P> pw[2];
  int psc[2];
  // tiles [0, n_clean) need no masking for any query of this wave
  int n_clean = S / KT;
  if (CAUSAL) n_clean = min(n_clean, (q_wave + 1) / KT);
  n_clean = min(n_clean, n_tiles);

  // Scores of chunk u of the tile in `base`: y = 2^23 s + start.  Masking
  // (keys past S, or above the diagonal) is applied by the epilogue on the
  // integer patterns, so masked tiles need no registers of their own.
  auto qk_chunk = [&](const uint8_t* base, int u) __attribute__((always_inline)) {
    const uint2 ksc = k_scales(base);
    if constexpr (KBATCH) {
    opv<F> kf[ND][2];
#pragma unroll
    for (int c = 0; c < ND; ++c)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) kf[c][bb] = kfrag(base, u, bb, c);
#pragma unroll
    for (int c = 0; c < ND; ++c)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int byte = u * 2 * ND + bb * ND + c;
        acc[u][bb] = mma32_sel<F>(kf[c][bb], qf[c], c == 0 ? minit : acc[u][bb],
                                  pick(ksc, byte), byte, qsc[c]);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * ND * (BITS == 4 ? 1 : 2) + 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * ND, 1);
    } else {
#pragma unroll
    for (int c = 0; c < ND; ++c)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int byte = u * 2 * ND + bb * ND + c;
        acc[u][bb] = mma32_sel<F>(kfrag(base, u, bb, c), qf[c], c == 0 ? minit : acc[u][bb],
                                  pick(ksc, byte), byte, qsc[c]);
      }
    }
  };
  // The exponential's bit pattern of register e of chunk u: the truncating
  // conversion of the product's output, or with the exact exponential the
  // vector unit's exp2 of t + R.  In a masked tile an invisible key's
  // pattern is set to 0 (P~ = 0), on the integer after the conversion.
  auto pattern = [&](int u, int e, int key0, int lim, auto masked_tag) __attribute__((always_inline)) {
    uint32_t pat;
    if constexpr (EXPX) pat = __float_as_uint(__builtin_amdgcn_exp2f(acc[u][e >> 4][e & 15]));
    else pat = cvt_u32_trunc(acc[u][e >> 4][e & 15]);
    if constexpr (decltype(masked_tag)::value) pat = key0 + ckey(u, e >> 4, e & 15) < lim ? pat : 0u;
    return pat;
  };
  // Bit-pattern exponential + MX quantisation of P for chunk u.  FP6/FP4:
  // the lane's 32 values are one whole block (keys 32h .. 32h+31 of the
  // chunk).  FP8: they are half of each of the chunk's two blocks (keys
  // 16h + i and 32 + 16h + i); one swap of the half maxima with the lane 32
  // apart gives every lane the maximum of block h, which it scales in the
  // P V product, and a second swap hands it the byte of the other block.
  // One scale per row (E4M3): every block takes the row's placement scale;
  // the row's largest pattern tells whether a value rounds beyond 448 (the
  // row then goes to the fallback pass; the products do not carry the NaN
  // codes of such values on).  Affine codes (E2M1): the code is
  // clamp(RNE(2 x + 2), 0, 7) of the exponent x relative to the block's
  // placement, formed from the product's output by one FMA and one
  // rounding conversion to a byte.
  auto epi = [&](int u, int key0, auto masked_tag) __attribute__((always_inline)) {
    const int lim = CAUSAL ? min(S, q + 1) : S;
    if constexpr (PM == PM_ROW) {
      float pv[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) pv[e] = __uint_as_float(pattern(u, e, key0, lim, masked_tag));
      constexpr int SB0 = 127 - PL;
      uint32_t w[8];
      Pack32<P, false>::run(pv, w, conv_scale(SB0), conv_scale(SB0));
#pragma unroll
      for (int i = 0; i < 8; ++i) pw[u][i] = (int)w[i];
      // The row overflows once a value reaches 464 (448 plus half its step:
      // it would round beyond 448), i.e. once a pattern reaches the bits of
      // 464 times the conversion's divisor.  Compared on the patterns as
      // integers: a row far above its guess has patterns at or past the
      // exponent field's top (NaN bit patterns, or the sign bit set), whose
      // converted codes need not show the overflow.
      auto uv = [&](int o) __attribute__((always_inline)) { return __float_as_uint(pv[o]); };
      uint32_t m0 = max(max(uv(0), uv(1)), uv(2));
      uint32_t m1 = max(max(uv(16), uv(17)), uv(18));
#pragma unroll
      for (int p = 3; p < 15; p += 2) {
        m0 = max(max(m0, uv(p)), uv(p + 1));
        m1 = max(max(m1, uv(16 + p)), uv(17 + p));
      }
      m0 = max(max(m0, uv(15)), max(m1, uv(31)));
      constexpr uint32_t OVER_BITS = __builtin_bit_cast(uint32_t, 464.0f * (float)(1ull << (REF - PL)));
      over |= m0 >= OVER_BITS ? 0x80u : 0u;
      psc[u] = SB0;
    } else if constexpr (PM == PM_EFQ) {
      float yv[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float y = acc[u][e >> 4][e & 15];
        if constexpr (decltype(masked_tag)::value) yv[e] = key0 + ckey(u, e >> 4, e & 15) < lim ? y : 0.0f;
        else yv[e] = y;
      }
      float m0 = __builtin_fmaxf(__builtin_fmaxf(yv[0], yv[1]), yv[2]);
      float m1 = __builtin_fmaxf(__builtin_fmaxf(yv[16], yv[17]), yv[18]);
#pragma unroll
      for (int p = 3; p < 15; p += 2) {
        m0 = __builtin_fmaxf(__builtin_fmaxf(m0, yv[p]), yv[p + 1]);
        m1 = __builtin_fmaxf(__builtin_fmaxf(m1, yv[16 + p]), yv[17 + p]);
      }
      m0 = __builtin_fmaxf(m0, yv[15]);
      m1 = __builtin_fmaxf(m1, yv[31]);
      const int x = block_binade<MB>(__builtin_fmaxf(m0, m1)) + 127 + REF;
      kmax = max(kmax, x);
      const int sb = min(max(x, XLO), XHI) - REF - PL;
      // 2 x_el + 2 = y 2^-22 - 2 (sb + REF) + 2, rounded and clamped to a byte
      const float kb = (float)(2 - 2 * (sb + REF));
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(yv[8 * wd + 2 * j], 0x1p-22f, kb), j, ev);
          od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(yv[8 * wd + 2 * j + 1], 0x1p-22f, kb), j, od);
        }
        pw[u][wd] = (int)(ev | (od << 4));
      }
      psc[u] = sb;
    } else {
      float pv[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int o = PBITS == 6 ? (e & 1) * 16 + (e >> 1) : e;   // FP6: evens, then odds
        pv[o] = __uint_as_float(pattern(u, e, key0, lim, masked_tag));
      }
      auto uv = [&](int o) __attribute__((always_inline)) { return __float_as_uint(pv[o]); };
      uint32_t m0 = max(max(uv(0), uv(1)), uv(2));
      uint32_t m1 = max(max(uv(16), uv(17)), uv(18));
#pragma unroll
      for (int p = 3; p < 15; p += 2) {
        m0 = max(max(m0, uv(p)), uv(p + 1));
        m1 = max(max(m1, uv(16 + p)), uv(17 + p));
      }
      m0 = max(m0, uv(15));
      m1 = max(m1, uv(31));
      uint32_t mb;
      if constexpr (PBITS == 8) {
        const auto hs = __builtin_amdgcn_permlane32_swap(m0, m1, false, false);
        mb = max((uint32_t)hs[0], (uint32_t)hs[1]);
      } else {
        mb = max(m0, m1);
      }
      const int x = block_level<MB>(mb);
      kmax = max(kmax, x);
      const int sb = min(max(x, XLO), XHI) - REF - PL;
      uint32_t w[8];
      if constexpr (PBITS == 8) {
        const auto sbs = __builtin_amdgcn_permlane32_swap((uint32_t)sb, (uint32_t)sb, false, false);
        Pack32<P, false>::run(pv, w, conv_scale((int)sbs[0]), conv_scale((int)sbs[1]));
      } else if constexpr (PBITS == 6) {
        pack_fp6_split<P>(pv, w, conv_scale(sb));
      } else {
        Pack32<P, false>::run(pv, w, conv_scale(sb), conv_scale(sb));
      }
#pragma unroll
      for (int i = 0; i < Operand<P>::words; ++i) pw[u][i] = (int)w[i];
      psc[u] = sb;
    }
  };

  auto pv_chunk = [&](const uint8_t* base, int u) __attribute__((always_inline)) {
    const uint2 vsc = v_scales(base);
    if constexpr (VBATCH) {
    opv<F> vf[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vf[db] = vfrag(base, u, db);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int byte = u * NDB + db;
      O[db] = mma32_pv_sel<F, P>(vf[db], pw[u], O[db], pick(vsc, byte), byte, psc[u]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NDB * (BITS == 4 ? 1 : 2) + 1, 2);
    __builtin_amdgcn_sched_group_barrier(0x008, NDB, 2);
    } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int byte = u * NDB + db;
      O[db] = mma32_pv_sel<F, P>(vfrag(base, u, db), pw[u], O[db], pick(vsc, byte), byte, psc[u]);
    }
    }
    if constexpr (L32)
      L = mfma32_v4_v8(ones, pw[u], L, Fmt<FMT_E2M1>::mfma, Fmt<P>::mfma, 0, 127, 0, psc[u]);
    else
      L = row_sum<P>(ones, pw[u], L, psc[u]);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // Tile t+1 lands while tile t is read; after the barrier that ends step t
  // its stages take tile t+2.
  // One tile in four phases split by fences: the scores of chunk 0; those of chunk 1
  // beside the epilogue of chunk 0; the P V products of chunk 0 beside the
  // epilogue of chunk 1; then those of chunk 1.  Left unfenced, the
  // scheduler interleaves further and lengthens live ranges until registers
  // spill (measured: every D=128 kernel spills, the FP8 one 335 registers),
  // and spill reloads do not mix safely with the LDS DMA in flight, whose
  // completions the compiler cannot see.  ALWAYS_ISSUE: the full-tile sweep
  // issues the load of step t+2 even past the last tile (it reloads the last
  // tile into a stage that is never read again), which keeps the sweep over
  // full tiles free of branches.
  auto step = [&](int t, auto st_tag, auto masked_tag, auto always_tag) __attribute__((always_inline)) {
    uint8_t* kb = kstage(st_tag);
    uint8_t* vb = vstage(st_tag);
    qk_chunk(kb, 0);
    __builtin_amdgcn_sched_barrier(0);
    qk_chunk(kb, 1);
    epi(0, t * KT, masked_tag);
    __builtin_amdgcn_sched_barrier(0);
    // The two waves on a SIMD come from different workgroups and drift
    // apart; raising this phase's priority lets its P V products and the
    // epilogue beside them win issue over the other wave's score phases
    // (measured: about +3 % for FP8/FP6, +6 % for FP4; raising the other
    // phases as well, or instead, gains less).
    __builtin_amdgcn_s_setprio(1);
    pv_chunk(vb, 0);
    epi(1, t * KT, masked_tag);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    pv_chunk(vb, 1);
    wait_dma();
    ring_barrier();
    if (decltype(always_tag)::value || t + 2 < n_tiles) {
      // past the last tile the full-tile sweep reloads the last one (its
      // stage is never read again): every load stays inside the slab, whose
      // range check does not cover the tile offset in the scalar operand
      const int tn = min(t + 2, n_tiles - 1);
      issue_k(tn, kb);
      issue_v(tn, vb);
    }
  };
  using F0 = std::false_type;
  using T1 = std::true_type;
  [[maybe_unused]] int kap_x = kap_in;
  if (REBASE && __syncthreads_or(kap_in >= KSAT)) {
    // scores-only sweep: the row's largest visible score, then the binade of
    // its value once rounded (the rule is monotone in the score), exact to
    // HI_BINADE (the bit patterns saturate far sooner)
    float tm = -INFINITY;
    const int lim = CAUSAL ? min(S, q + 1) : S;
    auto pstep = [&](int tt, auto st_tag) __attribute__((always_inline)) {
      uint8_t* kb = kstage(st_tag);
      qk_chunk(kb, 0);
      qk_chunk(kb, 1);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (tt * KT + ckey(u, bb, i) < lim) tm = __builtin_fmaxf(tm, acc[u][bb][i]);
      wait_dma();
      ring_barrier();
      if (tt + 2 < n_tiles) {
        issue_k(tt + 2, kb);
        issue_v(tt + 2, vstage(st_tag));
      }
    };
    for (int tt = 0; tt < n_tiles; tt += 2) {
      pstep(tt, I0{});
      if (tt + 1 < n_tiles) pstep(tt + 1, I1{});
    }
    tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32));
    int km;
    if constexpr (EXPX) {
      // the exact value 2^t rounds up a binade once 2^frac(t) >= 2 - 2^-(M+1)
      constexpr float F_UP = MB == 3 ? 0.95419631f : 0.80735492f;   // log2(1.9375), log2(1.75)
      const float t = tm - (float)REF;
      const float fl = __builtin_floorf(t);
      km = (int)__builtin_fminf(fl, (float)HI_BINADE) + (t - fl >= F_UP ? 1 : 0);
    } else {
      km = block_binade<MB>(tm, LO_PATTERN);
    }
    // a row far above its guess (km >= KSAT) or far below it (km < 0:
    // re-based downwards); the measure spans +-HI_BINADE
    kap_x = km;
    // restart the ring for the sweep from the raised reference
    issue_k(0, kl0);
    issue_v(0, vl0);
    wait_dma();
    __syncthreads();
    if (n_tiles > 1) { issue_k(1, kl1); issue_v(1, vl1); }
  }
  if constexpr (REBASE) {
    c0 = EXPX ? (float)(REF - kap_x) - mg
              : __builtin_fmaf(-8388608.0f, mg, 8388608.0f * (float)(127 + REF - kap_x));
#pragma unroll
    for (int i = 0; i < 16; ++i) minit[i] = c0;
  }
  int t = 0;
  // full tiles, two per iteration, branch-free
  for (; t + 1 < n_clean; t += 2) {
    step(t, I0{}, F0{}, T1{});
    step(t + 1, I1{}, F0{}, T1{});
  }
  // the rest: a last full tile and the masked tiles (t is even here)
  for (; t < n_tiles; t += 2) {
    if (t < n_clean) step(t, I0{}, F0{}, F0{});
    else step(t, I0{}, T1{}, F0{});
    if (t + 1 < n_tiles) step(t + 1, I1{}, T1{}, F0{});
  }

  // The full-tile sweep may have reloaded the last tile past the end; none
  // of those loads may still be writing this workgroup's LDS when the
  // workgroup ends and the LDS passes to the next one.
  wait_dma();

  // row offset in binades (the oracle's kappa); rows beyond EXT come out
  // wrong here and are recomputed by the REBASE pass
  int kap = kmax - (127 + REF);
  kap = max(kap, __shfl_xor(kap, 32));
  // a top block beyond the largest shift (the row more than CAP binades
  // below its guess, its scale clamped at XLO) is measured by the fallback
  // pass and re-based downwards, so that it still lands in the placement
  // binade; one scale per row has no block levels (its case is the zero
  // row sum below)
  if constexpr (PM != PM_ROW && !REBASE) kap = kap < -CAP ? KSAT : kap;
  kap = kap > 0 ? kap : 0;
  if constexpr (REBASE) kap = kap_x;
  // exact exponential: 2^(t + REF) leaves fp32's range (an infinite pattern)
  // from 128 - REF binades above the reference on, so larger offsets are
  // not known here; the fallback pass measures them
  if constexpr (EXPX && !REBASE) kap = kap >= 254 - (127 + REF) ? KSAT : kap;
  // row sum of query n: from the 32x32 product in every register of the
  // lane; from the 16x16 one, output row 0 of lane n (n < 16) or row 8 of
  // lane n + 16
  float lsum;
  if constexpr (L32) lsum = L[0];
  else lsum = __shfl(L[0], n < 16 ? n : n + 16);
  // one scale per row: a value past the format's range in either half of
  // the row sends it to the fallback pass, which measures its offset
  if constexpr (PM == PM_ROW && !REBASE) {
    const uint32_t ov = (over | (uint32_t)__shfl_xor((int)over, 32)) & 0x80u;
    kap = ov ? KSAT : 0;
  }
  // One scale per row: a row whose every code flushed to zero (a guess more
  // than the format's range above it: the row sum is 0) is measured by the
  // fallback pass too, and re-based downwards.
  if constexpr (PM == PM_ROW && !REBASE) kap = lsum == 0.0f ? KSAT : kap;

  // ---- normalise and store: register i of O[db] is d = 32 db + 8 (i/4) + 4h + i%4.
  // The row index is recomputed from an opaque lane index, so that the
  // prologue's copy (used to load Q) need not stay live across the sweep.
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int qe = q_wave + (lane_e & 31);
  const int he = lane_e >> 5;
  if (qe < S && (!REBASE || kap_in > EXT)) {
    // A key holding NaN or Inf (its K^ block scale is NaN) makes every score
    // against it NaN, which the truncating conversion would turn into a zero
    // probability: rows that see such a key are written NaN instead, as
    // softmax propagates it.  The quantiser recorded the first such key.
    const uint64_t nk = a.nan_key[wi];
    const bool poisoned = CAUSAL ? nk <= (uint64_t)qe : nk < (uint64_t)S;
    const float inv = poisoned ? __builtin_nanf("") : 1.0f / lsum;
    uint16_t* orow = a.out + b * a.o_sb + h * a.o_sh + (int64_t)qe * a.o_ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const uint32_t lo = f32_to_bf16_rne(O[db][4 * gq] * inv) |
                            ((uint32_t)f32_to_bf16_rne(O[db][4 * gq + 1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_rne(O[db][4 * gq + 2] * inv) |
                            ((uint32_t)f32_to_bf16_rne(O[db][4 * gq + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * gq + 4 * he) = make_uint2(lo, hi);
      }
    if (he == 0) a.row_kappa[(bh - a.row_bh0) * S + qe] = kap;
  }
  // tell the REBASE pass of this call that it has work (one vector store);
  // rows past S (a ragged last query tile) never ask for it
  if (!REBASE && __builtin_amdgcn_ballot_w64(qe < S && kap > EXT) != 0 && lane == 0)
    *a.fb_flag = a.call_id;
#endif  // __HIP_DEVICE_COMPILE__
}

// Byte i of a byte table in the kernel arguments, read as its aligned
// dword: a uniform index then gives a scalar load, which the constant cache
// serves, where a byte load went to memory and back before anything else.
__device__ __forceinline__ int table_byte(const uint8_t* t, int i) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(t)[i >> 2];
  return (int)((w >> (8 * (i & 3))) & 0xFFu);
}

// The attention kernel over the heads [h0, h0 + hrun) of every batch entry,
// each in its own element format from FSET (a bit set of FMT_*): one
// launch for a hybrid schedule.  PM is the P~ variant; PX picks a P~
// format other than the operands': 1 E4M3 over FP6/FP4, 2 E3M2 over E2M3.
// The format is uniform per workgroup, so the branch into its body is a
// scalar one.
template <int FSET, int PM, int PX, int D, bool CAUSAL, bool REBASE>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
fsa_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __align__(16) uint8_t kl0[attn_kstage_bytes(D)];
  __shared__ __align__(16) uint8_t kl1[attn_kstage_bytes(D)];
  __shared__ __align__(16) uint8_t vl0[attn_vstage_bytes(D)];
  __shared__ __align__(16) uint8_t vl1[attn_vstage_bytes(D)];
  constexpr int QW = 128;                    // queries per workgroup
  // XCD-aware work order: workgroup i runs on XCD i % 8; each XCD takes a
  // contiguous run of (batch entry, head slot, query tile) items so that
  // the workgroups sharing its L2 sweep the same head's K^ and V^.  Head
  // slots follow a.horder, which interleaves the formats of a hybrid
  // schedule so that every XCD gets its share of each.
  const int nq = (a.S + QW - 1) / QW;
  const int n_items = nq * a.B * a.hrun;
  const int per_xcd = (n_items + 7) / 8;
  // (The REBASE pass deals its items round-robin instead: its few busy
  // workgroups, often all from one head, then spread over every XCD.)
  const int item = REBASE ? (int)blockIdx.x : (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int bs = item / nq;                  // (batch entry, head slot)
  const int b = bs / a.hrun;
  const int j = table_byte(a.horder, bs - b * a.hrun);   // head within the launch
  const int64_t wi = (int64_t)b * a.hrun + j;
  // causal: a head's query tiles heaviest first (the last tile sees every
  // key), so that the light ones fill the end of the launch
  const int qi = item - bs * nq;
  const int q_wg = (CAUSAL && !REBASE ? nq - 1 - qi : qi) * QW;
  const int f = (FSET & (FSET - 1)) ? table_byte(a.hfmt, j) : 0;
  with_format<FSET>(f, [&](auto fc) {
    constexpr int FC = decltype(fc)::value;
    constexpr int PF = PX == 1 ? (int)FMT_E4M3 : PX == 2 ? (int)FMT_E3M2 : FC;
    attn_body<FC, PF, PM, D, CAUSAL, REBASE>(a, b, a.h0 + j, wi, q_wg, kl0, kl1, vl0, vl1);
  });
#endif  // __HIP_DEVICE_COMPILE__
}

// The two launches of one call's attention (sweep, then fallback pass).
template <int FSET, int PM, int PX, int D, bool CAUSAL>
hipError_t launch_attn3(const AttnArgs& a, hipStream_t stream) {
  constexpr int QW = 128;
  const int n_items = (a.S + QW - 1) / QW * a.B * a.hrun;
  dim3 grid((n_items + 7) / 8 * 8);
  hipLaunchKernelGGL((fsa_fwd_kernel<FSET, PM, PX, D, CAUSAL, false>), grid, dim3(256), 0, stream, a);
  // the fallback pass: ~4 us when the first pass left no row beyond EXT
  if (!a.skip_fallback)
    hipLaunchKernelGGL((fsa_fwd_kernel<FSET, PM, PX, D, CAUSAL, true>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int FSET, int PM, int PX>
hipError_t launch_attn2(const AttnArgs& a, int D, int causal, hipStream_t stream) {
  if (D == 128)
    return causal ? launch_attn3<FSET, PM, PX, 128, true>(a, stream) : launch_attn3<FSET, PM, PX, 128, false>(a, stream);
  return causal ? launch_attn3<FSET, PM, PX, 64, true>(a, stream) : launch_attn3<FSET, PM, PX, 64, false>(a, stream);
}

}  // namespace fsa
