// bwd.hip -- CKDA backward (placeholder until the kernels land).
#include "ckda_device.h"
#include "ckda_launch.h"

namespace ckda {

size_t bwd_workspace_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ckda
