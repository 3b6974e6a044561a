// Scan kernels with bfloat16 inputs (see scan_fwd_kernel.h).
#include "scan_fwd_kernel.h"

namespace ssm {
namespace fwd {
template hipError_t launch_variant<bf16_t, false>(const ScanArgs&, int, int, bool, hipStream_t);
}  // namespace fwd
}  // namespace ssm
