// Cache write (scatter new tokens into their slots) and copy-on-write block copy.
//
// [studynote 223] "KV Cache PagedAttention", section II figure: a growing request's
//   new KV is stored in whichever physical block its table links in next.
// [velog] "Paged Attention", section 작동 예시: tokens fill block after block.
// [studynote 223] section II copy-on-write paragraph; [velog] 메모리 공유
//   (Copy-on-Write): a shared block is duplicated before one sharer diverges.
//
// Both kernels move raw bits (16/32-bit integers), so every value -- NaN
// payloads included -- arrives unchanged.  At the sizes a decode step writes
// they are bound by launch and HBM latency.

#include <vector>

#include "pa_internal.h"

namespace pa {
namespace {

// One workgroup per (group of 8 new tokens, kv head).  Inside a block, K is
// stored as groups of W channels (32, or D when D is not a multiple of 32), each a run of bs token rows of W
// channels; consecutive threads take consecutive channels of one group, token
// after token, so the writes of consecutive slots are consecutive addresses.
// V is channel-major inside a block: a token's values are D elements bs apart.
// For V the threads are laid out token-fastest -- thread (c, i) stores token
// t0 + i of channels c, c + 32, ... -- so when the group's slots are
// consecutive (a prefill chunk, at any alignment) eight neighbouring threads
// write 8 neighbouring positions of one channel row, and their reads are 8
// neighbouring channels of one token row.
constexpr int kGroupTokens = 8;

// Workgroup -> (token group, kv head).  The grid is one-dimensional and
// remapped so that consecutive token groups of one head run on the same XCD:
// the groups of one block write disjoint 16-byte pieces of the same V channel
// rows, and when those pieces meet in one L2 they leave it as whole lines
// instead of partial writes from several XCDs.
__device__ __forceinline__ void group_and_head(int ngroups, int64_t* t0, int* g) {
    const int u = xcd_remap(blockIdx.x, gridDim.x);
    *g = u / ngroups;
    *t0 = static_cast<int64_t>(u % ngroups) * kGroupTokens;
}

template <typename W>   // W = uint16_t (bf16) or uint32_t (fp32): the element's bits
__global__ __launch_bounds__(256) void cache_write_kernel(
    W* __restrict__ kc, W* __restrict__ vc, const W* __restrict__ kn, const W* __restrict__ vn,
    const int64_t* __restrict__ slots, int32_t num_tokens, int32_t H, int32_t D, int32_t bs,
    int64_t num_slots) {
    int g;
    int64_t t0;
    group_and_head((num_tokens + kGroupTokens - 1) / kGroupTokens, &t0, &g);
    const int tid = threadIdx.x;
    const int nt = static_cast<int>(min(static_cast<int64_t>(kGroupTokens), num_tokens - t0));

    // K: channel group slowest, then token, then channel within the group
    const int GW = D % 32 == 0 ? 32 : D;          // channels per K group
    for (int e = tid; e < nt * D; e += 256) {
        const int grp = e / (nt * GW), i = (e / GW) % nt, dl = e % GW;
        const int d = grp * GW + dl;
        const int64_t slot = slots[t0 + i];
        if (slot < 0 || slot >= num_slots) continue;
        const int64_t blk = slot / bs, off = slot % bs;
        kc[(blk * H + g) * bs * D + (grp * static_cast<int64_t>(bs) + off) * GW + dl] =
            kn[((t0 + i) * H + g) * D + d];
    }
    // V: token-fastest
    const int i = tid % kGroupTokens;
    if (i >= nt) return;
    const int64_t slot = slots[t0 + i];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t blk = slot / bs, off = slot % bs;
    const W* src = vn + ((t0 + i) * H + g) * D;
    W* dst = vc + (blk * H + g) * D * static_cast<int64_t>(bs) + off;
    for (int d = tid / kGroupTokens; d < D; d += 256 / kGroupTokens)
        dst[static_cast<int64_t>(d) * bs] = src[d];
}

// The same scatter with 16-byte accesses, for head_dim a multiple of 32 (K
// rows then fall in whole 32-channel groups) and 16-byte-aligned buffers.  K:
// each thread moves one 16-byte piece of a token row straight to its group row;
// a wave moves four tokens, so consecutive slots give 256-byte runs.  V: the
// group's rows are staged in LDS with 16-byte loads, then stored token-fastest
// as in cache_write_kernel.  The slots are read once per workgroup.
template <typename W>
__global__ __launch_bounds__(256) void cache_write_vec_kernel(
    W* __restrict__ kc, W* __restrict__ vc, const W* __restrict__ kn, const W* __restrict__ vn,
    const int64_t* __restrict__ slots, int32_t num_tokens, int32_t H, int32_t D, int32_t bs,
    int64_t num_slots) {
    constexpr int EPV = 16 / sizeof(W);                    // elements per 16-byte piece
    __shared__ int64_t s_slot[kGroupTokens];
    __shared__ __align__(16) W s_v[kGroupTokens * 128 * 4 / sizeof(W)];   // D * sizeof(W) <= 512 bytes
    int g;
    int64_t t0;
    group_and_head((num_tokens + kGroupTokens - 1) / kGroupTokens, &t0, &g);
    const int tid = threadIdx.x;
    const int nt = static_cast<int>(min(static_cast<int64_t>(kGroupTokens), num_tokens - t0));
    const int pieces = D / EPV;                            // per token row
    if (tid < nt) s_slot[tid] = slots[t0 + tid];
    for (int e = tid; e < nt * pieces; e += 256) {
        const int i = e / pieces, p = e % pieces;
        *reinterpret_cast<uint4*>(&s_v[i * D + p * EPV]) =
            *reinterpret_cast<const uint4*>(&vn[((t0 + i) * H + g) * D + p * EPV]);
    }
    __syncthreads();
    for (int e = tid; e < nt * pieces; e += 256) {
        const int i = e / pieces, p = e % pieces;
        const int64_t slot = s_slot[i];
        if (slot < 0 || slot >= num_slots) continue;
        const int64_t blk = slot / bs, off = slot % bs;
        const int d0 = p * EPV;
        W* dst = kc + (blk * H + g) * bs * D + ((d0 >> 5) * static_cast<int64_t>(bs) + off) * 32 + (d0 & 31);
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&kn[((t0 + i) * H + g) * D + d0]);
    }
    const int i = tid % kGroupTokens;
    if (i >= nt) return;
    const int64_t slot = s_slot[i];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t blk = slot / bs, off = slot % bs;
    W* dst = vc + (blk * H + g) * D * static_cast<int64_t>(bs) + off;
    for (int d = tid / kGroupTokens; d < D; d += 256 / kGroupTokens) dst[static_cast<int64_t>(d) * bs] = s_v[i * D + d];
}

constexpr int kPairsPerLaunch = 128;

struct CopyBatch {
    int32_t src[kPairsPerLaunch];
    int32_t dst[kPairsPerLaunch];
};

// grid = (pairs in batch, 2 pools, splits of the block tile).  A (block, all
// heads) tile is contiguous in both pools; each workgroup copies 16-byte words
// [split * per_split, ...) of it.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ kc,
                                                          uint4* __restrict__ vc, CopyBatch b,
                                                          int64_t tile_words, int64_t per_split) {
    uint4* pool = blockIdx.y == 0 ? kc : vc;
    const int64_t src = static_cast<int64_t>(b.src[blockIdx.x]) * tile_words;
    const int64_t dst = static_cast<int64_t>(b.dst[blockIdx.x]) * tile_words;
    const int64_t lo = static_cast<int64_t>(blockIdx.z) * per_split;
    const int64_t hi = lo + per_split < tile_words ? lo + per_split : tile_words;
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) pool[dst + i] = pool[src + i];
}

}  // namespace
}  // namespace pa

extern "C" {

int pa_cache_write(void* k_cache, void* v_cache, const pa_cache_desc* desc, const void* k_new,
                   const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                   void* stream) {
    using namespace pa;
    if (!desc_ok(desc) || num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (desc->head_dim % 2) return PA_ERR_UNSUPPORTED;
    const int32_t H = desc->num_kv_heads, D = desc->head_dim, bs = desc->block_size;
    const int64_t num_slots = static_cast<int64_t>(desc->num_blocks) * bs;
    const int64_t groups = (static_cast<int64_t>(num_tokens) + kGroupTokens - 1) / kGroupTokens;
    if (groups * H > INT32_MAX) return PA_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<uint32_t>(groups * H));
    const bool aligned = ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
                           reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15) == 0;
    if (aligned && D % 32 == 0 && D <= 128) {
        if (desc->kv_dtype == PA_BF16)
            return launch_kernel(cache_write_vec_kernel<uint16_t>, grid, dim3(256), 0, st,
                                 static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                                 static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                 slot_mapping, num_tokens, H, D, bs, num_slots);
        return launch_kernel(cache_write_vec_kernel<uint32_t>, grid, dim3(256), 0, st,
                             static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                             static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new),
                             slot_mapping, num_tokens, H, D, bs, num_slots);
    }
    if (desc->kv_dtype == PA_BF16)
        return launch_kernel(cache_write_kernel<uint16_t>, grid, dim3(256), 0, st,
                             static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                             static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                             slot_mapping, num_tokens, H, D, bs, num_slots);
    return launch_kernel(cache_write_kernel<uint32_t>, grid, dim3(256), 0, st,
                         static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                         static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new),
                         slot_mapping, num_tokens, H, D, bs, num_slots);
}

int pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* desc,
                   const int64_t* pairs_host, int32_t n_pairs, void* stream) {
    using namespace pa;
    if (!desc_ok(desc) || n_pairs < 0) return PA_ERR_INVALID_ARG;
    if (n_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !pairs_host) return PA_ERR_INVALID_ARG;
    // 16-byte copies of whole (block, all heads) tiles
    if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % 16)
        return PA_ERR_INVALID_ARG;
    const int64_t N = desc->num_blocks;
    // Validate the whole list before launching anything: ids in range, no
    // destination twice, no destination that is also a source (so the copies
    // commute and may run concurrently).  One mark per block: O(n_pairs +
    // num_blocks) for any list.
    std::vector<uint8_t> is_dst;
    try {
        is_dst.assign(static_cast<size_t>(N), 0);
    } catch (...) {
        return PA_ERR_NO_MEMORY;
    }
    for (int32_t i = 0; i < n_pairs; ++i) {
        const int64_t s = pairs_host[2 * i], d = pairs_host[2 * i + 1];
        if (s < 0 || s >= N || d < 0 || d >= N) return PA_ERR_INVALID_ARG;
        if (is_dst[d]) return PA_ERR_INVALID_ARG;
        is_dst[d] = 1;
    }
    for (int32_t i = 0; i < n_pairs; ++i)
        if (is_dst[pairs_host[2 * i]]) return PA_ERR_INVALID_ARG;
    const int64_t tile_bytes = static_cast<int64_t>(desc->num_kv_heads) * desc->block_size *
                               desc->head_dim * static_cast<int64_t>(dtype_size(desc->kv_dtype));
    if (tile_bytes % 16) return PA_ERR_UNSUPPORTED;
    const int64_t tile_words = tile_bytes / 16;
    const int64_t per_split = 256 * 4;                          // 16 KB per workgroup
    const int64_t splits = (tile_words + per_split - 1) / per_split;
    if (splits > 65535) return PA_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t base = 0; base < n_pairs; base += kPairsPerLaunch) {
        const int32_t n = n_pairs - base < kPairsPerLaunch ? n_pairs - base : kPairsPerLaunch;
        CopyBatch b{};
        for (int32_t i = 0; i < n; ++i) {
            b.src[i] = static_cast<int32_t>(pairs_host[2 * (base + i)]);
            b.dst[i] = static_cast<int32_t>(pairs_host[2 * (base + i) + 1]);
        }
        const int rc = launch_kernel(copy_blocks_kernel, dim3(n, 2, static_cast<uint32_t>(splits)),
                                     dim3(256), 0, st, static_cast<uint4*>(k_cache),
                                     static_cast<uint4*>(v_cache), b, tile_words, per_split);
        if (rc != PA_OK) return rc;
    }
    return PA_OK;
}

}  // extern "C"
