// Backward launches for bf16 inputs and the dispatch over input element
// kinds (fp16 inputs: gdpa_bwd_f16.hip).
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int act_kind, int in_kind, bool want_dq, bool want_dkv,
                      hipStream_t stream) {
  switch (in_kind) {
    case EL_BF16: return launch_bwd_el<EL_BF16>(a, head_dim, act_kind, want_dq, want_dkv, stream);
    case EL_F16: return launch_bwd_f16(a, head_dim, act_kind, want_dq, want_dkv, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdpa
