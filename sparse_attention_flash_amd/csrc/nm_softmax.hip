// nm_softmax.hip -- N:M sparse softmax forward (gfx950).  Not implemented yet.
#include "kernels.h"
namespace sa {
hipError_t launch_nm_softmax(const NmArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sa
