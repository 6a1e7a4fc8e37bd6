// Forward launches for bf16 inputs, for FP8 and MXFP8 Q/K with bf16 V, and
// the dispatch over input element kinds (fp16 inputs: gdpa_fwd_f16.hip).
#include "gdpa_fwd.hpp"

namespace gdpa {

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int head_dim_v, int act_kind, int in_kind, hipStream_t stream) {
  switch (in_kind) {
    case EL_BF16: return launch_fwd_in<EL_BF16>(a, head_dim, head_dim_v, act_kind, stream);
    case EL_FP8: return launch_fwd_in<EL_FP8>(a, head_dim, head_dim_v, act_kind, stream);
    case EL_MX8: return launch_fwd_in<EL_MX8>(a, head_dim, head_dim_v, act_kind, stream);
    case EL_MX4: return launch_fwd_in<EL_MX4>(a, head_dim, head_dim_v, act_kind, stream);
    case EL_F16: return launch_fwd_f16(a, head_dim, head_dim_v, act_kind, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdpa
