// Fused-Softmax attention forward: E4M3 kernels.  One wave per SIMD (the FP8
// operands do not fit twice in the register file), so the accumulators may
// live in AGPRs, which leaves the architectural VGPRs to the software
// pipeline; this file is built without forcing the VGPR form of the MFMAs.
#include "fsa_fwd_impl.h"

namespace fsa {

hipError_t launch_fsa_fwd_e4m3(const AttnArgs& a, int D, int causal, hipStream_t stream) {
  return launch2<FMT_E4M3>(a, D, causal, stream);
}

}  // namespace fsa
