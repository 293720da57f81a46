#include "mala_device.h"
#include "mala_internal.h"
namespace mala {
hipError_t launch_bwd(const BwdParams&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
}
