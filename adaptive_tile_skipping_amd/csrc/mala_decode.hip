#include "mala_device.h"
#include "mala_internal.h"
namespace mala {
hipError_t launch_decode(const DecParams&, int, int, bool, hipStream_t) { return hipErrorNotSupported; }
}
