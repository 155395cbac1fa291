// P~ variants of the fused attention kernel (fsa_attn.h): one scale per row
// (E4M3), E4M3 P~ over FP6/FP4 operands, E3M2 P~ over E2M3 operands, and
// affine E2M1 codes.
#include "fsa_attn.h"

namespace fsa {

hipError_t launch_fsa_variant(const AttnArgs& a, int fset, int pm, int px, int D, int causal,
                              hipStream_t stream) {
  constexpr int E4 = 1 << FMT_E4M3, E6 = 1 << FMT_E2M3, E1 = 1 << FMT_E2M1;
  if (pm == PM_ROW && !px && fset == E4) return launch_attn2<E4, PM_ROW, 0>(a, D, causal, stream);
  if (pm == PM_EFQ && !px && fset == E1) return launch_attn2<E1, PM_EFQ, 0>(a, D, causal, stream);
  if (pm == PM_BLOCK && px == 2 && fset == E6) return launch_attn2<E6, PM_BLOCK, 2>(a, D, causal, stream);
  if (pm == PM_BLOCK && px == 1) {
    if (fset == E6) return launch_attn2<E6, PM_BLOCK, 1>(a, D, causal, stream);
    if (fset == E1) return launch_attn2<E1, PM_BLOCK, 1>(a, D, causal, stream);
    if (fset == (E6 | E1)) return launch_attn2<E6 | E1, PM_BLOCK, 1>(a, D, causal, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fsa
