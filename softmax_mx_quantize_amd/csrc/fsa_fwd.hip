// Fused-Softmax attention forward: E2M3 and E2M1 kernels and the dispatch.
// Built with the VGPR form of every MFMA: with two waves per SIMD the
// epilogue reads the score accumulators on the vector units, which cannot
// read AGPRs directly.
#include "fsa_fwd_impl.h"

namespace fsa {

hipError_t launch_fsa_fwd(const AttnArgs& a, int fmt, int D, int causal, hipStream_t stream) {
  if (fmt == FMT_E4M3) return launch_fsa_fwd_e4m3(a, D, causal, stream);
  if (fmt == FMT_E2M3) return launch2<FMT_E2M3>(a, D, causal, stream);
  return launch2<FMT_E2M1>(a, D, causal, stream);
}

}  // namespace fsa
