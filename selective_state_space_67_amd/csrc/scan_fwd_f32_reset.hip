// Scan kernels with float32 inputs and document resets (see scan_fwd_kernel.h).
#include "scan_fwd_kernel.h"

namespace ssm {
namespace fwd {
template hipError_t launch_variant<float, true>(const ScanArgs&, int, int, bool, hipStream_t);
}  // namespace fwd
}  // namespace ssm
