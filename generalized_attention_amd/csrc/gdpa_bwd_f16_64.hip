// Backward kernels for fp16 inputs (P and dS rounded to fp16) at head dim 64.
#include "gdpa_bwd.hpp"

namespace gdpa {

template hipError_t launch_bwd_ed<EL_F16, 64, 64>(const BwdArgs&, int, bool, bool, bool, hipStream_t);

}  // namespace gdpa
