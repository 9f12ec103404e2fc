// Internal helpers shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>

#include "../../include/pa.h"
#include "../../include/pa_measure.h"

namespace pa {

// ---- host-side validation -------------------------------------------------------
inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

inline size_t dtype_size(int32_t dt) { return dt == PA_F32 ? 4 : (dt == PA_BF16 ? 2 : 0); }

inline bool desc_ok(const pa_cache_desc* d) {
    return d && d->num_blocks > 0 && d->block_size > 0 && d->num_kv_heads > 0 &&
           d->head_dim > 0 && dtype_size(d->kv_dtype) != 0;
}

// Remember a failed HIP call's error code for pa_last_hip_error() (per thread)
// and return PA_ERR_HIP.  Defined in status.hip.
int record_hip_error(hipError_t e);

inline int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : record_hip_error(e); }

// Launch `kernel` and return the status of that launch alone.  The launch's
// own return code is used, never hipGetLastError(): the latter also reports
// errors left behind by unrelated HIP calls of the host program.  Arguments
// are converted to the kernel's parameter types first.  Does not synchronize.
// With start/stop events (either may be null) the launch goes through
// hipExtLaunchKernel, which records them at the start and the end of the
// kernel's own dispatch.
template <typename... KArgs, typename... Args>
int launch_kernel_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                        hipEvent_t start, hipEvent_t stop, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
    void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {};
    std::apply(
        [&ptrs](auto&... v) {
            int i = 0;
            ((ptrs[i++] = const_cast<void*>(static_cast<const void*>(&v))), ...);
        },
        vals);
    if (start || stop)
        return hip_status(hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds,
                                             st, start, stop, 0));
    return hip_status(
        hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, st));
}

template <typename... KArgs, typename... Args>
int launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                  Args... args) {
    return launch_kernel_timed(kernel, grid, block, lds, st, nullptr, nullptr, args...);
}

constexpr int kNumXcds = 8;   // MI355X: 8 XCDs, workgroups dispatched round-robin over them

// ---- device helpers ----------------------------------------------------------------
// Map a dispatch index to a work-unit index so that consecutive work units run
// on the same XCD (and so share its L2): dispatch id i goes to XCD i % 8; the
// units are dealt out so that XCD x receives one contiguous range of them.
// Bijective on [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int id, int n) {
    const int x = id % kNumXcds;
    const int k = id / kNumXcds;
    const int q = n / kNumXcds;
    const int r = n % kNumXcds;
    return x * q + (x < r ? x : r) + k;
}

}  // namespace pa
