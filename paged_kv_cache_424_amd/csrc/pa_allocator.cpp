// Host block allocator and block-table builder (pure C++17, no GPU).
//
// [velog] "Paged Attention", section 구현 세부사항 / 메모리 할당자: allocate_block()
//   hands out a free physical block, free_block(id) returns one for reuse.
// [studynote 223] "KV Cache PagedAttention", section II figure: a request grows by
//   linking an empty block into its table only when it needs room; [velog]
//   "작동 예시": at 16 tokens per block the new blocks come at tokens 1, 17, 33.
// [ch.09] "09. PagedAttention", section 해법: any free physical block can hold
//   the next logical block; waste is confined to the last block.
// [studynote 223] section II copy-on-write paragraph; [velog] 메모리 공유
//   (Copy-on-Write): requests with a common prefix share its blocks, and a
//   request that writes into a shared block first takes a private copy.
//
// Free list: FIFO ring over a fixed array (every block id appears at most once,
// so N slots suffice), seeded with the caller's order.  Reference counts per
// block.  Sequences live in a vector indexed by id; ids are never reused.
// Every call checks everything first and mutates only once it cannot fail.

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/pa.h"

namespace {

struct Sequence {
    bool alive = false;
    int64_t length = 0;
    std::vector<int32_t> blocks;   // logical order
};

}  // namespace

struct pa_allocator {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> ring;     // free list storage, capacity num_blocks
    int32_t head = 0;              // index of the first free block in ring
    int32_t count = 0;             // number of free blocks
    std::vector<int32_t> refcount;
    std::vector<Sequence> seqs;

    int32_t pop_free() {
        int32_t b = ring[head];
        head = (head + 1) % num_blocks;
        --count;
        refcount[b] = 1;
        return b;
    }
    void push_free(int32_t b) {
        ring[(head + count) % num_blocks] = b;
        ++count;
    }
    void drop_ref(int32_t b) {
        if (--refcount[b] == 0) push_free(b);
    }
    Sequence* seq(int32_t id) {
        if (id < 0 || id >= static_cast<int32_t>(seqs.size()) || !seqs[id].alive) return nullptr;
        return &seqs[id];
    }
    const Sequence* seq(int32_t id) const {
        if (id < 0 || id >= static_cast<int32_t>(seqs.size()) || !seqs[id].alive) return nullptr;
        return &seqs[id];
    }
    int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

extern "C" {

int pa_allocator_create(int32_t num_blocks, int32_t block_size,
                        const int32_t* initial_free_order, pa_allocator** out) {
    if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
    *out = nullptr;
    pa_allocator* a = new (std::nothrow) pa_allocator;
    if (!a) return PA_ERR_NO_MEMORY;
    try {
        a->num_blocks = num_blocks;
        a->block_size = block_size;
        a->ring.resize(num_blocks);
        a->refcount.assign(num_blocks, 0);
        if (initial_free_order) {
            std::vector<char> seen(num_blocks, 0);
            for (int32_t i = 0; i < num_blocks; ++i) {
                int32_t b = initial_free_order[i];
                if (b < 0 || b >= num_blocks || seen[b]) {
                    delete a;
                    return PA_ERR_INVALID_ARG;
                }
                seen[b] = 1;
                a->ring[i] = b;
            }
        } else {
            for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
        }
        a->head = 0;
        a->count = num_blocks;
    } catch (const std::bad_alloc&) {
        delete a;
        return PA_ERR_NO_MEMORY;
    }
    *out = a;
    return PA_OK;
}

void pa_allocator_destroy(pa_allocator* a) { delete a; }

int pa_allocate_block(pa_allocator* a, int32_t* block_out) {
    if (!a || !block_out) return PA_ERR_INVALID_ARG;
    if (a->count == 0) return PA_ERR_OUT_OF_BLOCKS;
    *block_out = a->pop_free();
    return PA_OK;
}

int pa_free_block(pa_allocator* a, int32_t block) {
    if (!a) return PA_ERR_INVALID_ARG;
    if (block < 0 || block >= a->num_blocks || a->refcount[block] == 0) return PA_ERR_BAD_BLOCK;
    a->drop_ref(block);
    return PA_OK;
}

int32_t pa_num_free(const pa_allocator* a) { return a ? a->count : PA_ERR_INVALID_ARG; }

int32_t pa_refcount(const pa_allocator* a, int32_t block) {
    if (!a) return PA_ERR_INVALID_ARG;
    if (block < 0 || block >= a->num_blocks) return PA_ERR_BAD_BLOCK;
    return a->refcount[block];
}

int pa_seq_create(pa_allocator* a, int32_t* seq_out) {
    if (!a || !seq_out) return PA_ERR_INVALID_ARG;
    if (a->seqs.size() >= static_cast<size_t>(INT32_MAX)) return PA_ERR_NO_MEMORY;
    try {
        a->seqs.emplace_back();
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;
    }
    a->seqs.back().alive = true;
    *seq_out = static_cast<int32_t>(a->seqs.size() - 1);
    return PA_OK;
}

int pa_seq_fork(pa_allocator* a, int32_t parent, int32_t* child_out) {
    if (!a || !child_out) return PA_ERR_INVALID_ARG;
    if (!a->seq(parent)) return PA_ERR_BAD_SEQ;
    try {
        Sequence child;
        child.alive = true;
        child.length = a->seqs[parent].length;
        child.blocks = a->seqs[parent].blocks;
        a->seqs.push_back(std::move(child));
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;
    }
    for (int32_t b : a->seqs.back().blocks) ++a->refcount[b];
    *child_out = static_cast<int32_t>(a->seqs.size() - 1);
    return PA_OK;
}

int pa_seq_append_slots(pa_allocator* a, int32_t seq, int32_t n_tokens,
                        int64_t* slot_mapping_out, int64_t* cow_pair_out, int32_t* n_cow_out) {
    if (!a || n_tokens < 0 || !n_cow_out || !cow_pair_out) return PA_ERR_INVALID_ARG;
    if (n_tokens > 0 && !slot_mapping_out) return PA_ERR_INVALID_ARG;
    Sequence* s = a->seq(seq);
    if (!s) return PA_ERR_BAD_SEQ;
    *n_cow_out = 0;
    if (n_tokens == 0) return PA_OK;
    const int64_t bs = a->block_size;
    const int64_t len = s->length;
    const bool needs_cow = (len % bs != 0) && a->refcount[s->blocks.back()] > 1;
    const int64_t new_blocks = a->blocks_for(len + n_tokens) - a->blocks_for(len);
    if (new_blocks + (needs_cow ? 1 : 0) > a->count) return PA_ERR_OUT_OF_BLOCKS;
    try {
        s->blocks.reserve(static_cast<size_t>(a->blocks_for(len + n_tokens)));
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;
    }
    if (needs_cow) {
        const int32_t src = s->blocks.back();
        const int32_t dst = a->pop_free();
        --a->refcount[src];                      // was > 1, stays >= 1
        s->blocks.back() = dst;
        cow_pair_out[0] = src;
        cow_pair_out[1] = dst;
        *n_cow_out = 1;
    }
    for (int64_t i = 0; i < n_tokens; ++i) {
        const int64_t p = len + i;
        if (p % bs == 0) s->blocks.push_back(a->pop_free());
        slot_mapping_out[i] = static_cast<int64_t>(s->blocks[p / bs]) * bs + p % bs;
    }
    s->length = len + n_tokens;
    return PA_OK;
}

int pa_seq_cow_block(pa_allocator* a, int32_t seq, int32_t logical_index, int64_t* cow_pair_out,
                     int32_t* n_cow_out) {
    if (!a || !cow_pair_out || !n_cow_out) return PA_ERR_INVALID_ARG;
    Sequence* s = a->seq(seq);
    if (!s) return PA_ERR_BAD_SEQ;
    if (logical_index < 0 || logical_index >= static_cast<int32_t>(s->blocks.size()))
        return PA_ERR_INVALID_ARG;
    *n_cow_out = 0;
    const int32_t src = s->blocks[logical_index];
    if (a->refcount[src] <= 1) return PA_OK;
    if (a->count == 0) return PA_ERR_OUT_OF_BLOCKS;
    const int32_t dst = a->pop_free();
    --a->refcount[src];
    s->blocks[logical_index] = dst;
    cow_pair_out[0] = src;
    cow_pair_out[1] = dst;
    *n_cow_out = 1;
    return PA_OK;
}

int pa_seq_free(pa_allocator* a, int32_t seq) {
    if (!a) return PA_ERR_INVALID_ARG;
    Sequence* s = a->seq(seq);
    if (!s) return PA_ERR_BAD_SEQ;
    for (int32_t b : s->blocks) a->drop_ref(b);
    s->alive = false;
    s->length = 0;
    std::vector<int32_t>().swap(s->blocks);
    return PA_OK;
}

int32_t pa_seq_length(const pa_allocator* a, int32_t seq) {
    if (!a) return PA_ERR_INVALID_ARG;
    const Sequence* s = a->seq(seq);
    if (!s) return PA_ERR_BAD_SEQ;
    if (s->length > INT32_MAX) return PA_ERR_UNSUPPORTED;
    return static_cast<int32_t>(s->length);
}

int pa_seq_block_table(const pa_allocator* a, int32_t seq, int32_t* table_out, int32_t cap,
                       int32_t* n_out) {
    if (!a || !n_out || cap < 0) return PA_ERR_INVALID_ARG;
    const Sequence* s = a->seq(seq);
    if (!s) return PA_ERR_BAD_SEQ;
    const int32_t n = static_cast<int32_t>(s->blocks.size());
    *n_out = n;
    if (n > cap || (n > 0 && !table_out)) return PA_ERR_INVALID_ARG;
    if (n) std::memcpy(table_out, s->blocks.data(), sizeof(int32_t) * n);
    return PA_OK;
}

int pa_build_block_tables(const pa_allocator* a, const int32_t* seqs, int32_t n,
                          int32_t max_blocks, int32_t* tables_out, int32_t* context_lens_out) {
    if (!a || n < 0 || max_blocks < 0) return PA_ERR_INVALID_ARG;
    if (n > 0 && (!seqs || !context_lens_out || (max_blocks > 0 && !tables_out)))
        return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        const Sequence* s = a->seq(seqs[i]);
        if (!s) return PA_ERR_BAD_SEQ;
        if (static_cast<int64_t>(s->blocks.size()) > max_blocks) return PA_ERR_INVALID_ARG;
        if (s->length > INT32_MAX) return PA_ERR_UNSUPPORTED;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Sequence* s = a->seq(seqs[i]);
        int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
        const int32_t nb = static_cast<int32_t>(s->blocks.size());
        for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < nb ? s->blocks[j] : -1;
        context_lens_out[i] = static_cast<int32_t>(s->length);
    }
    return PA_OK;
}

}  // extern "C"
