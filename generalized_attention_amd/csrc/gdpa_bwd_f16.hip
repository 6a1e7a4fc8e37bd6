// Backward launches for fp16 inputs (Q, K, V, dO fp16; P and dS rounded to fp16).
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_f16(const BwdArgs& a, int head_dim, int act_kind, bool want_dq, bool want_dkv,
                          hipStream_t stream) {
  return launch_bwd_el<EL_F16>(a, head_dim, act_kind, want_dq, want_dkv, stream);
}

}  // namespace gdpa
