// Internal helpers shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/pa.h"

namespace pa {

// ---- host-side validation -------------------------------------------------------
inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

inline size_t dtype_size(int32_t dt) { return dt == PA_F32 ? 4 : (dt == PA_BF16 ? 2 : 0); }

inline bool desc_ok(const pa_cache_desc* d) {
    return d && d->num_blocks > 0 && d->block_size > 0 && d->num_kv_heads > 0 &&
           d->head_dim > 0 && dtype_size(d->kv_dtype) != 0;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Launch-error check after a kernel launch (does not synchronize).
inline int launch_status() { return hip_status(hipGetLastError()); }

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
