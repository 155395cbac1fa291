// The fused attention kernel (fsa_attn.h) with the exact exponential: the
// vector unit's exp2 of the score in binades, so that P~ is 2^x rounded
// onto the element grid (the exact map's rounding thresholds).
#include "fsa_attn.h"

namespace fsa {

hipError_t launch_fsa_exp(const AttnArgs& a, int fset, int D, int causal, hipStream_t stream) {
  constexpr int E4 = 1 << FMT_E4M3, E6 = 1 << FMT_E2M3, E1 = 1 << FMT_E2M1;
  switch (fset) {
    case E4: return launch_attn2<E4, PM_EXP, 0>(a, D, causal, stream);
    case E6: return launch_attn2<E6, PM_EXP, 0>(a, D, causal, stream);
    case E1: return launch_attn2<E1, PM_EXP, 0>(a, D, causal, stream);
    case E6 | E1: return launch_attn2<E6 | E1, PM_EXP, 0>(a, D, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fsa
