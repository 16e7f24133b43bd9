#include "pa_device.h"
#include "pa_launch.h"
namespace pa {
hipError_t launch_prefill(const PrefillParams&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace pa
