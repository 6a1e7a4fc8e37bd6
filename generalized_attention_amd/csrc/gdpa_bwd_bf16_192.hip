// Backward kernels for bf16 inputs at head dims (192, 128) (Q and K 192, V 128).
#include "gdpa_bwd.hpp"

namespace gdpa {

template hipError_t launch_bwd_ed<EL_BF16, 192, 128>(const BwdArgs&, int, bool, bool, bool, hipStream_t);

}  // namespace gdpa
