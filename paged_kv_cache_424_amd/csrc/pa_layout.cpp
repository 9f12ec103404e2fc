// Host-side library calls: status names, version, pool size and the layout formula.
#include <cstdint>

#include "../../include/pa.h"

namespace {
bool desc_ok(const pa_cache_desc* d) {
    return d && d->num_blocks > 0 && d->block_size > 0 && d->num_kv_heads > 0 && d->head_dim > 0 &&
           (d->kv_dtype == PA_F32 || d->kv_dtype == PA_BF16);
}
}  // namespace

extern "C" {

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_OUT_OF_BLOCKS: return "out of free blocks";
        case PA_ERR_BAD_BLOCK: return "bad block id";
        case PA_ERR_BAD_SEQ: return "unknown sequence";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_UNSUPPORTED: return "unsupported shape";
        case PA_ERR_NO_MEMORY: return "host out of memory";
        case PA_ERR_TOO_LARGE: return "request exceeds a fixed limit of the library";
        default: return "unknown status";
    }
}

int32_t pa_version(void) { return (1 << 16) | 0; }

size_t pa_cache_pool_bytes(const pa_cache_desc* d) {
    if (!desc_ok(d)) return 0;
    const size_t es = d->kv_dtype == PA_F32 ? 4 : 2;
    return static_cast<size_t>(d->num_blocks) * d->num_kv_heads * d->block_size * d->head_dim * es;
}

int64_t pa_kv_offset(const pa_cache_desc* d, int32_t which, int64_t slot, int32_t head,
                     int32_t dim) {
    if (!desc_ok(d) || (which != 0 && which != 1)) return -1;
    const int64_t bs = d->block_size, H = d->num_kv_heads, D = d->head_dim;
    if (slot < 0 || slot >= static_cast<int64_t>(d->num_blocks) * bs || head < 0 || head >= H ||
        dim < 0 || dim >= D)
        return -1;
    const int64_t block = slot / bs, off = slot % bs;
    if (which == 0) {                                                   // groups of token rows
        const int64_t W = D % 32 == 0 ? 32 : D;
        return (block * H + head) * bs * D + ((dim / W) * bs + off) * W + dim % W;
    }
    return ((block * H + head) * D + dim) * bs + off;                   // channel rows
}

}  // extern "C"
