// The HIP error behind the most recent PA_ERR_HIP of the calling thread.
#include "pa_internal.h"

namespace pa {
namespace {
thread_local hipError_t g_last_hip_error = hipSuccess;
}  // namespace

int record_hip_error(hipError_t e) {
    g_last_hip_error = e;
    return PA_ERR_HIP;
}

}  // namespace pa

extern "C" {

int32_t pa_last_hip_error(void) { return static_cast<int32_t>(pa::g_last_hip_error); }

const char* pa_last_hip_error_name(void) { return hipGetErrorName(pa::g_last_hip_error); }

}  // extern "C"
