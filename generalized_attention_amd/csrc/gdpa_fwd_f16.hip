// Forward launches for fp16 inputs (Q, K, V fp16; P rounded to fp16).
#include "gdpa_fwd.hpp"

namespace gdpa {

hipError_t launch_fwd_f16(const FwdArgs& a, int head_dim, int head_dim_v, int act_kind, hipStream_t stream) {
  return launch_fwd_in<EL_F16>(a, head_dim, head_dim_v, act_kind, stream);
}

}  // namespace gdpa
