/*
 * pa.h -- C ABI of the paged KV cache library for MI355X (gfx950).
 *
 * A KV cache stored in fixed-size physical blocks that need not be contiguous,
 * reached through a per-sequence block table, with blocks handed out on demand
 * and shared between sequences with copy-on-write.  Pages this follows:
 *
 *   [studynote 223] "KV Cache PagedAttention" (agnusdei1207 brainscience study note 223)
 *   [studynote 528] "vLLM PagedAttention KV cache optimization" (agnusdei1207 study note 528)
 *   [ch.09]         "09. PagedAttention" (119-ai-studio LLM inference guide, chapter 9)
 *   [velog]         "Paged Attention" (velog.io/@junegood)
 *
 * Conventions for every call:
 *   - Return value: PA_OK (0) or a negative pa_status.  Nothing is printed and no
 *     C++ exception crosses this boundary.
 *   - Host-side calls (allocator, sizes, layout) touch no GPU and may run on a
 *     machine without one.
 *   - Device calls take DEVICE pointers the caller owns (allocated by the caller,
 *     e.g. through torch); the library never allocates or frees device memory.
 *     They are asynchronous on `stream` (a hipStream_t; NULL = the null stream),
 *     never synchronize, and return PA_ERR_HIP if a launch fails.  Arguments that
 *     live on the host are validated before anything is launched; values that
 *     live on the device (block tables, lengths, slots) are bounds-checked by the
 *     kernels, which never read or write outside the buffers described here.
 *   - The calling thread's current HIP device is the one used.
 *
 * Cache layout (both pools are flat arrays of the cache dtype; H = kv heads,
 * bs = block_size, D = head_dim, W = 32 channels per K group when D is a
 * multiple of 32, else W = D; slot s is token offset s % bs of block s / bs):
 *   K pool element (block b, head g, offset o, channel d) at
 *       (b*H + g)*bs*D + ((d / W)*bs + o)*W + d % W
 *   V pool element (block b, head g, offset o, channel d) at ((b*H + g)*D + d)*bs + o
 * so one (block, head) tile is contiguous in each pool: K as D/W groups of bs
 * token rows of W channels, V as D channel rows of bs tokens.  pa_kv_offset()
 * evaluates this.
 *
 * Calls that measure the library rather than perform the method (kernel
 * timing, the plain streaming-read yardstick) are declared in pa_measure.h.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,   /* a pointer, size or shape is invalid */
    PA_ERR_OUT_OF_BLOCKS = -2, /* the pool has too few free blocks; nothing changed */
    PA_ERR_BAD_BLOCK = -3,     /* block id out of range or not allocated */
    PA_ERR_BAD_SEQ = -4,       /* unknown sequence id */
    PA_ERR_HIP = -5,           /* a HIP runtime call or kernel launch failed */
    PA_ERR_UNSUPPORTED = -6,   /* valid, but a shape the library has no kernel for */
    PA_ERR_NO_MEMORY = -7,     /* host allocation failed */
    PA_ERR_TOO_LARGE = -8      /* the call needs more than a fixed limit of the library */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Shape of one paged cache (one layer): num_blocks physical blocks of
 * block_size token slots, num_kv_heads heads of head_dim channels, stored as
 * kv_dtype (a pa_dtype). */
typedef struct pa_cache_desc {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t kv_dtype;
} pa_cache_desc;

/* ---- library ---------------------------------------------------------------- */

/* Human-readable name of a pa_status value (static storage). */
const char* pa_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int32_t pa_version(void);

/* The hipError_t value behind the most recent PA_ERR_HIP returned on the
 * calling thread (hipSuccess = 0 if there was none), and its name as HIP
 * spells it (static storage).  Launches are checked through their own return
 * code, so an error left pending by unrelated HIP calls is never reported. */
int32_t pa_last_hip_error(void);
const char* pa_last_hip_error_name(void);

/* ---- layout (host) ----------------------------------------------------------- */

/* Bytes of ONE pool (K or V) for this shape; 0 if desc is invalid. */
size_t pa_cache_pool_bytes(const pa_cache_desc* desc);

/* Element offset of (slot, head, dim) in the K pool (which = 0) or the V pool
 * (which = 1), per the layout above.  -1 for an invalid argument.  The physical
 * block of a slot is a design freedom the pages leave open ([ch.09] "해법":
 * any free physical block may hold a logical block); the arrangement inside a
 * block is this library's. */
int64_t pa_kv_offset(const pa_cache_desc* desc, int32_t which, int64_t slot, int32_t head,
                     int32_t dim);

/* ---- block allocator (host) ----------------------------------------------------
 * [velog] "구현 세부사항 / 메모리 할당자": allocate_block() returns a free physical
 * block id and free_block(id) returns a block for reuse.  [studynote 223]
 * section II figure and [velog] "작동 예시": a sequence takes a new block only when
 * its last block is full (tokens 1, 17, 33, ... at 16 tokens per block).
 * [studynote 223] section II copy-on-write paragraph and [velog] "메모리 공유
 * (Copy-on-Write)": sequences with a common prefix share its blocks; a writer
 * into a shared block first gets a private copy.
 *
 * Rules of this implementation: the free list is FIFO, seeded with
 * initial_free_order (NULL = 0..N-1); a block whose reference count drops to
 * zero goes to its tail.  Every call is all-or-nothing.  Sequence ids are
 * 0, 1, 2, ... in creation order and never reused.  An allocator is not
 * thread-safe; distinct allocators are independent.  All outputs go to
 * caller-owned host memory. */
typedef struct pa_allocator pa_allocator;

/* Create an allocator over num_blocks blocks of block_size tokens.
 * initial_free_order: NULL or a permutation of 0..num_blocks-1 (copied).
 * *out receives the handle (library-owned; release with pa_allocator_destroy). */
int pa_allocator_create(int32_t num_blocks, int32_t block_size,
                        const int32_t* initial_free_order, pa_allocator** out);
void pa_allocator_destroy(pa_allocator* a);

/* The pages' allocate_block(): pop the head of the free list, count = 1. */
int pa_allocate_block(pa_allocator* a, int32_t* block_out);
/* The pages' free_block(): drop one reference; at zero the block is free again.
 * PA_ERR_BAD_BLOCK if the block is out of range or not allocated. */
int pa_free_block(pa_allocator* a, int32_t block);
/* Number of free blocks (>= 0), or a negative status. */
int32_t pa_num_free(const pa_allocator* a);
/* Reference count of a block (>= 0), or a negative status. */
int32_t pa_refcount(const pa_allocator* a, int32_t block);

/* New empty sequence. */
int pa_seq_create(pa_allocator* a, int32_t* seq_out);
/* New sequence sharing every block of `parent` (each block's count + 1). */
int pa_seq_fork(pa_allocator* a, int32_t parent, int32_t* child_out);
/* Grow `seq` by n_tokens (>= 0).  slot_mapping_out[i] (n_tokens entries, may be
 * NULL when n_tokens == 0) receives the slot of position length+i, where
 * slot = physical_block * block_size + position % block_size.  If the last
 * block is partially filled and shared, it is first replaced by a fresh block
 * and the pair (src, dst) is written to cow_pair_out[0..1]; *n_cow_out is 1 then,
 * else 0.  The caller must copy src to dst (pa_copy_blocks) before writing the
 * new tokens.  PA_ERR_OUT_OF_BLOCKS leaves everything unchanged. */
int pa_seq_append_slots(pa_allocator* a, int32_t seq, int32_t n_tokens,
                        int64_t* slot_mapping_out, int64_t* cow_pair_out, int32_t* n_cow_out);
/* Make logical block `logical_index` of `seq` private: if it is shared, a
 * fresh block replaces it and (src, dst) is written to cow_pair_out with
 * *n_cow_out = 1; otherwise nothing changes and *n_cow_out = 0. */
int pa_seq_cow_block(pa_allocator* a, int32_t seq, int32_t logical_index,
                     int64_t* cow_pair_out, int32_t* n_cow_out);
/* Automatic prefix caching ([studynote 528] section II key ideas and section
 * IV: requests with the same system prompt share its blocks instead of
 * recomputing them; [ch.09] closing section: finding reusable prompt blocks
 * automatically).  Must be called before any block is allocated or sequence
 * created (else PA_ERR_INVALID_ARG).  From then on:
 *   - a full block's content is identified exactly by (the content of the
 *     block before it, its block_size token ids);
 *   - a block that fills with known content (through pa_seq_append_tokens) is
 *     registered as the cached block of that content, unless one already is;
 *   - a registered block whose count drops to zero keeps its contents on an
 *     evictable list (oldest first) instead of returning to the free list;
 *   - every allocation (pa_allocate_block, appends, copies) takes the free
 *     list's head, else evicts the oldest evictable block. */
int pa_allocator_enable_prefix_cache(pa_allocator* a);
/* Number of evictable cached blocks (>= 0), or a negative status. */
int32_t pa_num_cached(const pa_allocator* a);
/* Grow `seq` by n_tokens tokens whose ids are token_ids[0..n_tokens-1].  As
 * pa_seq_append_slots, except that with prefix caching on, each new block the
 * call fills completely, in a sequence whose content is known, is looked up:
 * if a block with the same content is cached, the sequence points at it (its
 * count + 1) and slot_mapping_out holds -1 for its tokens -- their K/V is
 * already in the pool, and pa_cache_write skips negative slots.
 * *n_cached_out receives the number of such tokens.  Cache hits are taken
 * before any fresh block of the call is allocated.  pa_seq_append_slots (no
 * token ids) makes the sequence's content unknown: none of its later blocks
 * is looked up or registered.  Without prefix caching this is
 * pa_seq_append_slots with *n_cached_out = 0.  PA_ERR_OUT_OF_BLOCKS leaves
 * everything unchanged. */
int pa_seq_append_tokens(pa_allocator* a, int32_t seq, const int32_t* token_ids, int32_t n_tokens,
                         int64_t* slot_mapping_out, int64_t* cow_pair_out, int32_t* n_cow_out,
                         int32_t* n_cached_out);
/* Release every block of `seq` (logical order) and forget the sequence. */
int pa_seq_free(pa_allocator* a, int32_t seq);
/* Tokens held by `seq` (>= 0), or a negative status. */
int32_t pa_seq_length(const pa_allocator* a, int32_t seq);
/* Copy the block table of `seq` into table_out (capacity `cap` entries);
 * *n_out receives its length.  PA_ERR_INVALID_ARG if cap is too small. */
int pa_seq_block_table(const pa_allocator* a, int32_t seq, int32_t* table_out, int32_t cap,
                       int32_t* n_out);
/* Block tables of n sequences as an int32 [n][max_blocks] row-major array padded
 * with -1, plus their lengths in context_lens_out[n].  PA_ERR_INVALID_ARG if a
 * sequence holds more than max_blocks blocks. */
int pa_build_block_tables(const pa_allocator* a, const int32_t* seqs, int32_t n,
                          int32_t max_blocks, int32_t* tables_out, int32_t* context_lens_out);

/* Occupancy of the pool, for capacity and fragmentation accounting.  The
 * pages contrast the waste of reserving one contiguous region per request at
 * its maximum length (internal fragmentation: slots reserved and never
 * filled; external: free space cut into pieces too small to use) with paging,
 * where waste is confined to the unfilled tail of each sequence's last block
 * ([ch.09] "문제: 연속 할당의 단편화" and "해법: 페이지처럼 나눠 담기";
 * [velog] "메모리 낭비 (Internal Fragmentation)").  Exact counts:
 *   num_blocks     pool size;
 *   free_blocks    blocks on the free list;
 *   cached_blocks  count-0 blocks kept for prefix reuse (evictable);
 *   used_blocks    blocks with count >= 1; shared_blocks: count >= 2;
 *   live_seqs      sequences created and not freed;
 *   logical_tokens sum of the live sequences' lengths;
 *   stored_tokens  slots of used blocks that hold a token of some live
 *                  sequence, each physical slot counted once however many
 *                  sequences share it (slot o of block b is held when a
 *                  sequence with b at logical index i has length > i*bs + o);
 *   hit_tokens     tokens pa_seq_append_tokens found cached, since creation;
 *   evictions      cached blocks handed to a new owner, since creation.
 * So used_blocks*block_size - stored_tokens slots are allocated and empty,
 * and sharing saves logical_tokens - stored_tokens slots.  Costs O(num_blocks
 * + table entries); PA_ERR_NO_MEMORY if host scratch cannot be allocated. */
typedef struct {
    int32_t num_blocks, free_blocks, cached_blocks, used_blocks, shared_blocks, live_seqs;
    int64_t logical_tokens, stored_tokens, hit_tokens, evictions;
} pa_allocator_stats;
int pa_allocator_get_stats(const pa_allocator* a, pa_allocator_stats* out);

/* ---- device operations ------------------------------------------------------------ */

/* Scatter new tokens into their cache slots ([studynote 223] section II figure:
 * a growing request's new KV goes into the block the table links in;
 * [velog] "작동 예시").
 *   k_cache, v_cache: device pools (layout above), written.
 *   k_new, v_new:     device [num_tokens][num_kv_heads][head_dim], cache dtype.
 *   slot_mapping:     device int64 [num_tokens]; a negative slot is padding and
 *                     writes nothing; a slot >= num_blocks*block_size is ignored.
 *                     The non-negative slots must be distinct (the allocator
 *                     never hands out a slot twice): if two tokens name the same
 *                     slot, the tokens' stores race and the slot may end up
 *                     holding elements of either.
 * Bit-exact copy: no arithmetic is applied to the values. */
int pa_cache_write(void* k_cache, void* v_cache, const pa_cache_desc* desc, const void* k_new,
                   const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                   void* stream);

/* Copy-on-write block copy ([studynote 223] section II copy-on-write paragraph;
 * [velog] "메모리 공유 (Copy-on-Write)"): for each pair, every head and slot of
 * block src is copied to block dst, in both pools.
 *   pairs_host: HOST int64 [n_pairs][2] = (src, dst), as the allocator emits them.
 *   k_cache, v_cache: 16-byte aligned.
 * PA_ERR_INVALID_ARG (nothing launched) if an id is out of range, a dst repeats,
 * a dst is also a src, or a pool is misaligned; the check costs O(n_pairs +
 * num_blocks) host time and num_blocks bytes of host memory (PA_ERR_NO_MEMORY
 * if those cannot be had).  The ids travel in kernel arguments, so the call
 * makes no host-to-device copy and needs no workspace. */
int pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* desc,
                   const int64_t* pairs_host, int32_t n_pairs, void* stream);

/* Workspace bytes pa_decode needs: room for the running max, sum and
 * unnormalised output of every piece of every (sequence, query head), plus one
 * piece count per (sequence, query head).  With fixed partitions
 * (partition_size > 0) a head has ceil(L / partition_size) pieces and no
 * workspace is needed (0) while max_context_len fits one partition; with the
 * balanced split (partition_size 0) a head of n 32-token chunks has at most
 * ceil(n / 4) + 1 pieces.  0 also for invalid arguments. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/* Paged decode attention: one query token per sequence against its context,
 * read block by block through its block table ([studynote 223] three-line summary
 * item 3 and section II: attention over scattered blocks bound by the table;
 * [ch.09] "해법": logical blocks look contiguous, physical ones are scattered).
 * For query head h the result is softmax(scale * K q_h) V over positions
 * 0..context_lens[s]-1 of kv head h / (num_q_heads / num_kv_heads).
 *   out:          device [num_seqs][num_q_heads][head_dim] of out_dtype (PA_F32 or PA_BF16).
 *   q:            device [num_seqs][num_q_heads][head_dim] in the cache dtype.
 *   q, k_cache, v_cache: 16-byte aligned (PA_ERR_INVALID_ARG otherwise).
 *   block_tables: device int32 [num_seqs][max_blocks_per_seq]; only the first
 *                 ceil(L/block_size) entries of a row are read.
 *   context_lens: device int32 [num_seqs]; L counts the newest token.
 *   max_context_len: an upper bound of every L, used to size the grid.
 *   partition_size: 0 for the balanced split -- the 32-token chunks of all
 *                 (sequence, kv head) pairs, each pair charged two chunks more
 *                 for starting a piece, are cut into equal ranges, one per
 *                 workgroup the chip holds at once, so the cut points (and the
 *                 fp32 rounding order of a row) depend on the whole batch and
 *                 the device's compute-unit count; or P > 0, a multiple of 32,
 *                 for pieces at absolute positions 0, P, 2P, ..., which make a
 *                 row's result depend on that row alone.
 *   workspace:    device scratch of >= pa_decode_workspace_bytes(...) bytes
 *                 (8-byte aligned), or NULL when that is 0.  Its contents
 *                 before the call do not matter.  Calls that overlap in time
 *                 must not share a workspace.
 * Device-side checks: a row whose L is < 1 or > max_context_len, whose needed
 * table entries leave [0, num_blocks), or whose L exceeds
 * max_blocks_per_seq*block_size, produces NaN outputs instead of reading out of
 * bounds.  Supported: head_dim 64 or 128, num_q_heads/num_kv_heads in 1..16,
 * block_size 8..256 a power of two, cache PA_F32 or PA_BF16.  PA_ERR_UNSUPPORTED
 * for anything else, and for a partition_size that is not a multiple of 32.
 * Runs pa_decode_partitions then pa_decode_reduce. */
int pa_decode(void* out, int32_t out_dtype, const void* q, const void* k_cache,
              const void* v_cache, const pa_cache_desc* desc, const int32_t* block_tables,
              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
              void* workspace, size_t workspace_bytes, void* stream);

/* First half of pa_decode: the split-K pass.  Heads whose context is a single
 * piece get their final output written here; the others leave per-piece
 * partials and their piece count in the workspace for pa_decode_reduce.
 * Same arguments and checks as pa_decode. */
int pa_decode_partitions(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                         const void* v_cache, const pa_cache_desc* desc,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_context_len, float scale, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Second half of pa_decode: merge the pieces of every (sequence, query head)
 * that has more than one, rescaling each piece's sum and output by
 * exp(its max - overall max).  Arguments as in pa_decode (the same values must
 * be passed to both halves); context_lens is not read (the piece counts come
 * from the workspace) and may be NULL. */
int pa_decode_reduce(void* out, int32_t out_dtype, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                     int32_t partition_size, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Decode with append: the decode step of sequences whose newest token
 * (position context_lens[s] - 1) has just been produced, in one pass instead of
 * pa_cache_write followed by pa_decode ([studynote 223] section II figure: the
 * new token's KV goes into the block its table links in, and the request then
 * attends over all its blocks).  The newest tokens are stored at
 * slot_mapping[s] of the pools by the workgroups that attend over the
 * sequences' last chunks, which then read them back with the rest of the
 * context (a workgroup-scope release/acquire orders the two).
 *   k_new, v_new:  device [num_seqs][num_kv_heads][head_dim], cache dtype,
 *                  aligned to their element.
 *   slot_mapping:  device int64 [num_seqs]: the slot the allocator gave position
 *                  context_lens[s] - 1 of sequence s.  Negative: nothing is
 *                  stored (as pa_cache_write, the attention then reads whatever
 *                  the pool holds there); a slot >= num_blocks*block_size is
 *                  ignored.
 *   k_cache, v_cache: written at those slots, read everywhere.
 * Other arguments, checks and results as pa_decode: the output and the pools
 * equal those of pa_cache_write(k_new, v_new, slot_mapping) + pa_decode bit
 * for bit, provided no row of the call reads a slot that another row stores
 * (copy-on-write in the allocator guarantees this: a new token never lands in
 * a block another sequence reads).  A row whose context length is invalid
 * (NaN output) stores nothing.
 * PA_ERR_INVALID_ARG if k_new, v_new or slot_mapping is NULL with num_seqs > 0,
 * or misaligned. */
int pa_decode_append(void* out, int32_t out_dtype, const void* q, const void* k_new,
                     const void* v_new, const int64_t* slot_mapping, void* k_cache, void* v_cache,
                     const pa_cache_desc* desc, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t max_context_len, float scale,
                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/* First half of pa_decode_append (the split-K pass with the append); pair it
 * with pa_decode_reduce as for pa_decode_partitions. */
int pa_decode_append_partitions(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                const void* v_new, const int64_t* slot_mapping, void* k_cache,
                                void* v_cache, const pa_cache_desc* desc,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_context_len, float scale,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream);

/* pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and results as pa_decode with the same arguments, but the
 * split-K workspace is a fixed array inside the library
 * (PA_DECODE_NO_ALLOC_MAX_WORKSPACE bytes per device, held from the first call
 * on a device until the process ends) instead of caller memory.  The call
 * allocates nothing; the caller still passes q, the pools, tables, lengths and
 * out.  PA_ERR_TOO_LARGE (nothing launched) when
 * pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
 * partition_size) exceeds the limit: with 512-token partitions, for instance,
 * 240 sequences x 64 query heads x 8,192 tokens at head_dim 128 fit.  Every
 * call on one device shares that device's array (its contents before a call do
 * not matter): calls that overlap in time on one device -- on different
 * streams, or from different host threads -- race and must not be made. */
#define PA_DECODE_NO_ALLOC_MAX_WORKSPACE ((size_t)128 << 20)
int pa_decode_no_alloc(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                       const void* v_cache, const pa_cache_desc* desc, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t max_context_len, float scale,
                       int32_t partition_size, void* stream);

/* Causal attention of prefill chunks over their paged context, the prefill half
 * of a continuous-batching step ([studynote 223] section IV checklist item 2;
 * [studynote 528] section II, continuous batching table).
 *   q:                device [num_query_tokens][num_q_heads][head_dim] (cache dtype),
 *                     the queries of all chunks back to back; chunk c owns rows
 *                     query_start_loc[c] .. query_start_loc[c+1]-1.
 *   q, k_cache, v_cache: 16-byte aligned (PA_ERR_INVALID_ARG otherwise).
 *   query_start_loc:  device int32 [num_chunks+1], non-decreasing, within
 *                     [0, num_query_tokens].
 *   context_lens:     device int32 [num_chunks]; L_c counts the chunk's own tokens,
 *                     which must already be in the cache as its last C_c positions.
 *                     Query i of the chunk sits at position L_c - C_c + i and sees
 *                     positions 0..L_c - C_c + i.
 *   block_tables:     device int32 [num_chunks][max_blocks_per_seq].
 *   max_query_len:    upper bound of every C_c (grid sizing).
 *   out:              device [num_query_tokens][num_q_heads][head_dim] of out_dtype;
 *                     rows that belong to no chunk are not written.
 * Device-side checks: the rows of a chunk with C_c < 0, C_c > max_query_len,
 * L_c < C_c, L_c > max_blocks_per_seq*block_size or a needed table entry
 * outside [0, num_blocks) are set to NaN (when they lie inside the output), and
 * nothing is read out of bounds.  Supported: bf16 cache, head_dim 128,
 * num_q_heads/num_kv_heads a power of two up to 16, block_size 8..256 a power
 * of two, one block of all kv heads (num_kv_heads x block_size x 256 bytes)
 * below 4 GiB.  scale must be finite and > 0 (PA_ERR_INVALID_ARG otherwise): the
 * running maximum is kept on the unscaled logits.  The value pass takes the
 * softmax weights in bf16 (fp32 accumulate), and each row's weight sum is taken
 * from the same bf16 weights. */
int pa_prefill(void* out, int32_t out_dtype, const void* q, const void* k_cache,
               const void* v_cache, const pa_cache_desc* desc, const int32_t* block_tables,
               int32_t max_blocks_per_seq, const int32_t* context_lens,
               const int32_t* query_start_loc, int32_t num_chunks, int32_t num_query_tokens,
               int32_t num_q_heads, int32_t max_query_len, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
