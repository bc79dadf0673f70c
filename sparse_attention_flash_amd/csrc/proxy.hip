// proxy.hip -- proxy-compensated block-sparse forward (gfx950).  Not implemented yet.
#include "kernels.h"
namespace sa {
hipError_t launch_proxy(const ProxyArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sa
