// Backward kernels for bf16 inputs at head dim 64.
#include "gdpa_bwd.hpp"

namespace gdpa {

template hipError_t launch_bwd_ed<EL_BF16, 64, 64>(const BwdArgs&, int, bool, bool, bool, hipStream_t);

}  // namespace gdpa
