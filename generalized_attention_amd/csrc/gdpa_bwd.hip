// Backward dispatch over input element kinds and head dims; the kernels of
// each (kind, head dim) are instantiated in gdpa_bwd_<type>_<dim>.hip.
#include "gdpa_bwd.hpp"

namespace gdpa {

template <int EL>
static hipError_t launch_bwd_el(const BwdArgs& a, int head_dim, int act_kind, bool want_dq, bool want_dkv, bool fused,
                                hipStream_t stream) {
  if (head_dim == 64) return launch_bwd_ed<EL, 64>(a, act_kind, want_dq, want_dkv, fused, stream);
  if (head_dim == 96) return launch_bwd_ed<EL, 96>(a, act_kind, want_dq, want_dkv, fused, stream);
  if (head_dim == 128) return launch_bwd_ed<EL, 128>(a, act_kind, want_dq, want_dkv, fused, stream);
  if (head_dim == 192) return launch_bwd_ed<EL, 192, 128>(a, act_kind, want_dq, want_dkv, fused, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int act_kind, int in_kind, bool want_dq, bool want_dkv,
                      bool fused, hipStream_t stream) {
  switch (in_kind) {
    case EL_BF16: return launch_bwd_el<EL_BF16>(a, head_dim, act_kind, want_dq, want_dkv, fused, stream);
    case EL_F16: return launch_bwd_el<EL_F16>(a, head_dim, act_kind, want_dq, want_dkv, fused, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdpa
