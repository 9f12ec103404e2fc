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
//
// Automatic prefix caching (optional, [studynote 528] section II key ideas and
// section IV: requests with the same system prompt share its blocks and skip
// recomputing it; [ch.09] closing section: finding reusable prompt blocks is
// the next step after paging).  A full block's content is identified exactly
// by (the content id of the block before it, its block_size token ids); ids
// are handed out 1, 2, ... and 0 is the empty prefix.  A block that fills with
// known content is registered as the cached block of that content.  When its
// reference count drops to zero, a registered block moves to an evictable
// list (oldest first) with its contents intact instead of to the free list;
// allocation takes a free block first and otherwise evicts the oldest
// evictable one.  pa_seq_append_tokens looks each new full block up and, on a
// hit, points the sequence at the cached block and reports slot -1 for its
// tokens (their K/V is already in the pool).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <iterator>
#include <list>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

struct Sequence {
    bool alive = false;
    int64_t length = 0;
    std::vector<int32_t> blocks;   // logical order
    int64_t chain = 0;             // content id of the last full block; -1: content unknown
    std::vector<int32_t> pending;  // token ids of the partial last block (content known)
};

struct ContentKey {
    int64_t parent;
    std::vector<int32_t> tokens;
    bool operator<(const ContentKey& o) const {
        return parent != o.parent ? parent < o.parent : tokens < o.tokens;
    }
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
    // prefix caching
    bool caching = false;
    std::map<ContentKey, int64_t> content_ids;
    std::unordered_map<int64_t, int32_t> cached;   // content id -> registered block
    std::vector<int64_t> content_of;               // block -> content id, 0 if not registered
    std::list<int32_t> evictable;                  // registered blocks with count 0, oldest first
    std::vector<std::list<int32_t>::iterator> evict_pos;
    std::vector<char> in_evictable;
    // cumulative counters for the occupancy statistics
    int64_t hit_tokens = 0;
    int64_t evictions = 0;

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
    int64_t available() const { return count + static_cast<int64_t>(evictable.size()); }
    // A block for a new owner: the free list's head, else the oldest evictable
    // block, which forgets its content.  The caller has checked available().
    int32_t take_block() {
        if (count > 0) return pop_free();
        const int32_t b = evictable.front();
        evictable.pop_front();
        in_evictable[b] = 0;
        ++evictions;
        cached.erase(content_of[b]);
        content_of[b] = 0;
        refcount[b] = 1;
        return b;
    }
    // One more owner of a cached block (taking it off the evictable list).
    void take_cached(int32_t b) {
        if (refcount[b] == 0 && in_evictable[b]) {
            evictable.erase(evict_pos[b]);
            in_evictable[b] = 0;
        }
        ++refcount[b];
    }
    void drop_ref(int32_t b) {
        if (--refcount[b] != 0) return;
        if (content_of[b] != 0) {
            evictable.push_back(b);
            evict_pos[b] = std::prev(evictable.end());
            in_evictable[b] = 1;
        } else {
            push_free(b);
        }
    }
    // Content id of (parent, tokens); 0 when absent and create is false.
    int64_t content(int64_t parent, const int32_t* tok, int32_t n, bool create) {
        ContentKey k{parent, std::vector<int32_t>(tok, tok + n)};
        auto it = content_ids.find(k);
        if (it != content_ids.end()) return it->second;
        if (!create) return 0;
        const int64_t id = static_cast<int64_t>(content_ids.size()) + 1;
        content_ids.emplace(std::move(k), id);
        return id;
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
        a->content_of.assign(num_blocks, 0);
        a->evict_pos.resize(num_blocks);
        a->in_evictable.assign(num_blocks, 0);
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

int pa_allocator_enable_prefix_cache(pa_allocator* a) {
    if (!a) return PA_ERR_INVALID_ARG;
    if (!a->seqs.empty() || a->count != a->num_blocks) return PA_ERR_INVALID_ARG;
    a->caching = true;
    return PA_OK;
}

int32_t pa_num_cached(const pa_allocator* a) {
    return a ? static_cast<int32_t>(a->evictable.size()) : PA_ERR_INVALID_ARG;
}

int pa_allocate_block(pa_allocator* a, int32_t* block_out) {
    if (!a || !block_out) return PA_ERR_INVALID_ARG;
    if (a->available() == 0) return PA_ERR_OUT_OF_BLOCKS;
    *block_out = a->take_block();
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
        child.chain = a->seqs[parent].chain;
        child.pending = a->seqs[parent].pending;
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
    if (new_blocks + (needs_cow ? 1 : 0) > a->available()) return PA_ERR_OUT_OF_BLOCKS;
    try {
        s->blocks.reserve(static_cast<size_t>(a->blocks_for(len + n_tokens)));
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;
    }
    // tokens of unknown content: none of this sequence's later blocks can be
    // looked up or registered
    s->chain = -1;
    s->pending.clear();
    if (needs_cow) {
        const int32_t src = s->blocks.back();
        const int32_t dst = a->take_block();
        --a->refcount[src];                      // was > 1, stays >= 1
        s->blocks.back() = dst;
        cow_pair_out[0] = src;
        cow_pair_out[1] = dst;
        *n_cow_out = 1;
    }
    for (int64_t i = 0; i < n_tokens; ++i) {
        const int64_t p = len + i;
        if (p % bs == 0) s->blocks.push_back(a->take_block());
        slot_mapping_out[i] = static_cast<int64_t>(s->blocks[p / bs]) * bs + p % bs;
    }
    s->length = len + n_tokens;
    return PA_OK;
}

int pa_seq_append_tokens(pa_allocator* a, int32_t seq, const int32_t* token_ids, int32_t n_tokens,
                         int64_t* slot_mapping_out, int64_t* cow_pair_out, int32_t* n_cow_out,
                         int32_t* n_cached_out) {
    if (!a || n_tokens < 0 || !n_cow_out || !cow_pair_out || !n_cached_out) return PA_ERR_INVALID_ARG;
    if (n_tokens > 0 && (!slot_mapping_out || !token_ids)) return PA_ERR_INVALID_ARG;
    *n_cached_out = 0;
    if (!a->caching)
        return pa_seq_append_slots(a, seq, n_tokens, slot_mapping_out, cow_pair_out, n_cow_out);
    Sequence* s = a->seq(seq);
    if (!s) return PA_ERR_BAD_SEQ;
    *n_cow_out = 0;
    if (n_tokens == 0) return PA_OK;
    const int64_t bs = a->block_size;
    const int64_t len = s->length;
    const int64_t end = len + n_tokens;
    const bool needs_cow = (len % bs != 0) && a->refcount[s->blocks.back()] > 1;
    // ---- plan: which of the new blocks are found in the cache ----
    std::vector<std::pair<int64_t, int32_t>> hits;   // (logical block, cached block)
    int64_t new_blocks = 0, pinned = 0;
    try {
        s->blocks.reserve(static_cast<size_t>(a->blocks_for(end)));
        s->pending.reserve(static_cast<size_t>(bs));
        int64_t chain = s->chain;
        std::vector<int32_t> pend = s->pending;
        for (int64_t p = len; p < end;) {
            const int64_t i = p - len;
            if (p % bs == 0) {
                ++new_blocks;
                const bool full = p + bs <= end;
                if (full && chain >= 0) {
                    const int64_t cid = a->content(chain, token_ids + i, static_cast<int32_t>(bs), false);
                    if (cid != 0) {
                        auto it = a->cached.find(cid);
                        if (it != a->cached.end()) {
                            hits.emplace_back(p / bs, it->second);
                            if (a->refcount[it->second] == 0) ++pinned;
                        }
                    }
                    chain = a->content(chain, token_ids + i, static_cast<int32_t>(bs), true);
                }
                p += full ? bs : end - p;
            } else {
                const int64_t take = std::min<int64_t>(bs - p % bs, end - p);
                if (chain >= 0) {
                    pend.insert(pend.end(), token_ids + i, token_ids + i + take);
                    if (static_cast<int64_t>(pend.size()) == bs) {
                        chain = a->content(chain, pend.data(), static_cast<int32_t>(bs), true);
                        pend.clear();
                    }
                }
                p += take;
            }
        }
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;
    }
    const int64_t fresh = new_blocks - static_cast<int64_t>(hits.size()) + (needs_cow ? 1 : 0);
    if (fresh > a->available() - pinned) return PA_ERR_OUT_OF_BLOCKS;
    // ---- execute: hits first, then the copy-on-write block, then fresh blocks ----
    for (const auto& h : hits) a->take_cached(h.second);
    if (needs_cow) {
        const int32_t src = s->blocks.back();
        const int32_t dst = a->take_block();
        --a->refcount[src];
        s->blocks.back() = dst;
        cow_pair_out[0] = src;
        cow_pair_out[1] = dst;
        *n_cow_out = 1;
    }
    size_t hi = 0;
    int32_t n_cached = 0;
    int64_t chain = s->chain;
    std::vector<int32_t>& pend = s->pending;
    // Every content id this loop needs was created by the plan and every
    // vector is reserved; only registering a block can allocate (a map node).
    try {
    for (int64_t p = len; p < end; ++p) {
        const int64_t lb = p / bs;
        const bool hit = hi < hits.size() && hits[hi].first == lb;
        if (p % bs == 0) s->blocks.push_back(hit ? hits[hi].second : a->take_block());
        if (hit) {
            slot_mapping_out[p - len] = -1;
            ++n_cached;
        } else {
            slot_mapping_out[p - len] = static_cast<int64_t>(s->blocks[lb]) * bs + p % bs;
        }
        if (chain >= 0) {
            pend.push_back(token_ids[p - len]);
            if (static_cast<int64_t>(pend.size()) == bs) {
                chain = a->content(chain, pend.data(), static_cast<int32_t>(bs), true);
                pend.clear();
                const int32_t b = s->blocks[lb];
                if (a->cached.find(chain) == a->cached.end()) {   // register (a hit is already)
                    a->cached.emplace(chain, b);
                    a->content_of[b] = chain;
                }
            }
        }
        if (hit && (p + 1) % bs == 0) ++hi;
    }
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;   // host memory exhausted while registering a block
    }
    s->length = end;
    s->chain = chain;
    if (chain < 0) pend.clear();
    a->hit_tokens += n_cached;
    *n_cached_out = n_cached;
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
    if (a->available() == 0) return PA_ERR_OUT_OF_BLOCKS;
    const int32_t dst = a->take_block();
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
    std::vector<int32_t>().swap(s->pending);
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

int pa_allocator_get_stats(const pa_allocator* a, pa_allocator_stats* out) {
    if (!a || !out) return PA_ERR_INVALID_ARG;
    pa_allocator_stats st{};
    st.num_blocks = a->num_blocks;
    st.free_blocks = a->count;
    st.cached_blocks = static_cast<int32_t>(a->evictable.size());
    for (int32_t b = 0; b < a->num_blocks; ++b) {
        st.used_blocks += a->refcount[b] >= 1;
        st.shared_blocks += a->refcount[b] >= 2;
    }
    // filled[b]: slots of block b below the longest reach of any holder
    std::vector<int32_t> filled;
    try {
        filled.assign(a->num_blocks, 0);
    } catch (const std::bad_alloc&) {
        return PA_ERR_NO_MEMORY;
    }
    const int64_t bs = a->block_size;
    for (const Sequence& s : a->seqs) {
        if (!s.alive) continue;
        ++st.live_seqs;
        st.logical_tokens += s.length;
        for (size_t i = 0; i < s.blocks.size(); ++i) {
            const int64_t reach = std::min<int64_t>(bs, s.length - static_cast<int64_t>(i) * bs);
            int32_t& f = filled[s.blocks[i]];
            if (reach > f) f = static_cast<int32_t>(reach);
        }
    }
    for (int32_t f : filled) st.stored_tokens += f;
    st.hit_tokens = a->hit_tokens;
    st.evictions = a->evictions;
    *out = st;
    return PA_OK;
}

}  // extern "C"
