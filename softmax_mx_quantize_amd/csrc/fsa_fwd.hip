// Fused-Softmax attention forward for MXFP8 (E4M3), MXFP6 (E2M3) and MXFP4
// (E2M1) operands on the 32x32x64 scaled MFMA of gfx950: the default P~
// (per-block scales, bit-pattern exponential) for every set of formats,
// the dispatch to the P~ variants (fsa_fwd_var.hip, fsa_fwd_exp.hip), and
// the debug view of the prologue's Q' operands.  The kernel itself is in
// fsa_attn.h.
#include "fsa_attn.h"

namespace fsa {

hipError_t launch_fsa_variant(const AttnArgs& a, int fset, int pm, int px, int D, int causal,
                              hipStream_t stream);
hipError_t launch_fsa_exp(const AttnArgs& a, int fset, int D, int causal, hipStream_t stream);

hipError_t launch_fsa_fwd(const AttnArgs& a, int fset, int pm, int px, int D, int causal,
                          hipStream_t stream) {
  if (pm == PM_EXP) return launch_fsa_exp(a, fset, D, causal, stream);
  if (pm != PM_BLOCK || px) return launch_fsa_variant(a, fset, pm, px, D, causal, stream);
  switch (fset) {
    case 1 << FMT_E4M3: return launch_attn2<1 << FMT_E4M3, PM_BLOCK, 0>(a, D, causal, stream);
    case 1 << FMT_E2M3: return launch_attn2<1 << FMT_E2M3, PM_BLOCK, 0>(a, D, causal, stream);
    case 1 << FMT_E2M1: return launch_attn2<1 << FMT_E2M1, PM_BLOCK, 0>(a, D, causal, stream);
    case (1 << FMT_E2M3) | (1 << FMT_E2M1):
      return launch_attn2<(1 << FMT_E2M3) | (1 << FMT_E2M1), PM_BLOCK, 0>(a, D, causal, stream);
    default: return launch_attn2<7, PM_BLOCK, 0>(a, D, causal, stream);
  }
}

namespace {

// One wave per 32 query rows, lanes laid out as in the attention kernel's
// prologue (lane (h, n) = 32 h + n holds D block 2c + h of query n for each
// 64-wide D chunk c); each lane writes its operand bytes and scale byte back
// in the public row layout.
template <int F, int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(64, 64))) q_operand_dump_kernel(QDumpArgs a) {
  constexpr int BITS = Fmt<F>::bits;
  constexpr int ND = D / 64, NDB = D / 32, RB = D * BITS / 8;
  const int lane = threadIdx.x;
  const int hh = lane >> 5, n = lane & 31;
  const int64_t r = (int64_t)blockIdx.x * 32 + n;
  const bool live = r < a.rows;
  const uint16_t* qrow = a.q + (live ? r : a.rows - 1) * D;
#pragma unroll
  for (int c = 0; c < ND; ++c) {
    int sc = 0;
    const int blk = 2 * c + hh;
    int col[4];
    uint4 qw[4];
    if constexpr (BITS == 8) q_cols32(c, hh, col);
    else q_cols(blk, col);
    q_words(qrow, live, col, qw);
    if constexpr (BITS == 8) {
      const v8i o = q_operand32_e4m3<23>(qw, a.qmul, hh, sc);
      if (live) {
        uint8_t* row = a.codes + r * RB;
        *reinterpret_cast<uint4*>(row + 64 * c + 16 * hh) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(row + 64 * c + 32 + 16 * hh) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    } else {
      const opv<F> o = q_operand<F, 23>(qw, a.qmul, sc);
      if (live) {
        uint8_t* dst = a.codes + r * RB + blk * 4 * BITS;
        if constexpr (BITS == 6) {
          uint2* d2 = reinterpret_cast<uint2*>(dst);
          d2[0] = make_uint2(o[0], o[1]);
          d2[1] = make_uint2(o[2], o[3]);
          d2[2] = make_uint2(o[4], o[5]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
    if (live) a.scales[r * NDB + blk] = (uint8_t)sc;
  }
}

template <int F>
hipError_t launch_q_dump_fmt(const QDumpArgs& a, int D, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + 31) / 32));
  if (D == 128) hipLaunchKernelGGL((q_operand_dump_kernel<F, 128>), grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL((q_operand_dump_kernel<F, 64>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q_operand_dump(const QDumpArgs& a, int fmt, int D, hipStream_t stream) {
  if (fmt == FMT_E4M3) return launch_q_dump_fmt<FMT_E4M3>(a, D, stream);
  if (fmt == FMT_E2M3) return launch_q_dump_fmt<FMT_E2M3>(a, D, stream);
  return launch_q_dump_fmt<FMT_E2M1>(a, D, stream);
}

}  // namespace fsa
