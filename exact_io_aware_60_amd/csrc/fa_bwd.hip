// fa_bwd.hip -- backward pass (kernels to follow).
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    (void)p; (void)stream;
    return hipErrorNotSupported;
}
}  // namespace fa
