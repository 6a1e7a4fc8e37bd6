// Fused backward kernels (dK, dV and dQ in one pass) for fp16 inputs at head dim 128.
#include "gdpa_bwd.hpp"

namespace gdpa {

template hipError_t launch_bwd_fused_ed<EL_F16, 128>(const BwdArgs&, int, hipStream_t);

}  // namespace gdpa
