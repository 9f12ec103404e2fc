// Paged decode attention for gfx950: a persistent split-K kernel plus a
// rescaling reduce.
//
// What is computed: for every sequence s and query head h, attention of the
// one new query over the sequence's whole context, read block by block through
// its block table ([studynote 223] "KV Cache PagedAttention", three-line summary
// item 3 and section II figure; [ch.09] "09. PagedAttention", section 해법: the
// request sees contiguous logical blocks, the blocks themselves are scattered).
// Paging changes where K/V live, not the result, so the kernels must reach
// softmax(scale * K q) V of the gathered context.
//
// Work split.  The context of one (sequence, kv head) is cut into pieces; each
// piece yields a partial (running max m, sum l, unnormalised output o) per
// query head of the group, and the reduce kernel merges the pieces.  A head
// whose context is a single piece gets its final output directly.  Two ways
// to cut:
//   * balanced (partition_size == 0, the default): the (sequence, kv head,
//     32-token chunk) space is laid end to end and cut into equal ranges, one
//     per workgroup, so every workgroup streams about the same number of
//     bytes whatever the length mix.  A range may cover the tail of one
//     (sequence, head), several short ones and the head of the next.  Each
//     (sequence, head) is charged two chunk slots more than it has chunks:
//     the slots stand for what starting a piece costs (the query load, the
//     first block-id window, the merge and the partial store), so a range
//     that starts many pieces streams fewer chunks (measured: 3.7 % faster on
//     a lognormal batch of 240, 5.7 % on a uniform batch of 64).  Where the cuts fall
//     depends on every length in the batch (and on the number of compute
//     units), so a row's rounding may change with the rest of the batch.
//     The grid is persistent: as many workgroups as the chip holds at once.
//     Each first reads every context length into LDS and scans them, so no
//     workgroup is spent on an empty partition and no host-side length is
//     needed.
//   * fixed partitions (partition_size = P > 0): pieces start at absolute
//     positions 0, P, 2P, ...; a row's result depends on its own length only.
//     One workgroup per (sequence, kv head, partition), dispatched by the
//     hardware as slots free up, which suits batches of similar lengths.
// Scheduling is static on purpose: handing out work through an atomic
// counter measured 30-45 % slower on this chip, where device-scope atomics on
// one word from all eight XCDs take microseconds each.

// Inside a partition.  The four waves take its 32-token chunks round robin, in
// windows of 16 chunks (512 tokens) whose block ids are staged in LDS (double
// buffered, one barrier per window).  Each wave keeps an online softmax per
// query head and the four waves are merged through LDS at the end.  In the
// balanced split the merged results of a workgroup's pieces wait in LDS (up
// to 24 KB) and are stored together when that buffer is full and at the end
// of the range: a wave's memory counter retires stores and loads in order,
// and under the saturating read stream a store issued between two pieces held
// up the next piece's first load wait until it was acknowledged (measured:
// 4-5 % faster on a lognormal batch of 240, bit-identical results).
//
// Matrix cores.  The query group (G <= 16 heads) against a 16-token K tile is
// a dense contraction, done as S^T[token][head] = K[token][:] . Q^T with
// v_mfma_f32_16x16x32_bf16 (fp32: v_mfma_f32_16x16x4_f32).  The value pass is
// done transposed too, O^T[channel][head] = V^T[channel][token] . P^T, so that
// (a) a lane's softmax weights are exactly the B operand it needs -- lane
// (j, r) holds head r's weights of tokens 8j..8j+7 of the chunk -- and (b) the
// per-head rescale of the running output is lane-local (columns are heads).
// The K tile rows are permuted (row r of tile t is token 8(r/4) + r%4 + 4t) to
// line the QK output up with that operand.  K is stored in 32-channel groups
// inside a block (each group a run of token rows of 64 bytes), so one load
// instruction of a k-group reads runs of four adjacent tokens: 256 contiguous
// bytes, whole cache lines (token rows of all D channels would give each
// instruction half of 16 different lines; measured 3-4 % slower).  V is stored
// channel-major inside a block so that the 8 consecutive tokens of one
// channel are one 16-byte load.
// bf16 weights are fed to the value MFMA as a hi + lo pair of bf16 numbers, so
// the product keeps ~16 bits of the fp32 weight (one extra MFMA per step; the
// kernel is bound by HBM, not by the matrix cores).
//
// A result depends on logical positions and lengths only, never on physical
// block ids, and no atomics are used: outputs are bit-identical under any
// relabelling of blocks and whether a prefix is shared or duplicated.

#include <algorithm>
#include <atomic>
#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 32;                              // tokens per wave step
constexpr int kMinBlock = 8;                            // smallest supported block size
constexpr int kMaxSeqsPerLaunch = 1024;                 // lengths scanned in LDS per launch
constexpr int kMinPieceChunks = 4;                      // balanced: at least 128 tokens per range
constexpr int kPieceSlots = 2;                           // balanced: chunk slots charged per (sequence, head)
constexpr int kMergeHeads = 8;                          // heads merged per LDS pass (12-wave groups)
constexpr int kPendFloats = 6144;                       // balanced: LDS floats of merged pieces held back
constexpr int kPendSlots = 8;                           // balanced: pieces held back at most

// Waves per SIMD the kernel is held to (register budget) and waves per
// workgroup: fixed partitions use 4-wave workgroups, the balanced split one
// workgroup that fills a CU (4 SIMDs x waves per SIMD).
template <bool BF16, int D>
constexpr int waves_per_simd() { return BF16 || D == 64 ? 3 : 2; }
template <bool BF16, int D, bool FIXED>
constexpr int waves_per_group() { return 4; }

struct DecodeArgs {
    void* out;
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* tables;
    const int32_t* lens;
    float* ws_acc;     // [B][Hq][pmax][D]
    float2* ws_ml;     // [B][Hq][pmax] (max in log2 units, sum)
    int32_t* ws_np;    // [B][Hq] pieces of the (sequence, head)
    // Decode with append (all null otherwise): the newest token (position L - 1)
    // of sequence s has K/V k_new[s], v_new[s] ([B][H][D], cache dtype); they
    // are used for that position and stored at slot new_slots[s] of kw / vw.
    const void* k_new;
    const void* v_new;
    const int64_t* new_slots;
    void* kw;
    void* vw;
    int32_t B, Hq, H, G, bs, N, maxb, max_ctx;
    int32_t part_chunks;   // > 0: fixed partitions of this many 32-token chunks; 0: balanced
    int32_t pmax;          // piece slots per (sequence, head) in the workspace
    float scale_log2;      // scale * log2(e): logits are kept in base-2 units
    int32_t out_bf16;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, int out_bf16) {
    if (out_bf16)
        static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);
    else
        static_cast<float*>(out)[idx] = v;
}

// Zero the 16-bit lanes of a uint4 (8 bf16 tokens) whose token index is >= n.
__device__ __forceinline__ u32x4 keep_first_bf16(u32x4 v, int n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (2 * e < n) ? 0x0000ffffu : 0u;
        const uint32_t hi = (2 * e + 1 < n) ? 0xffff0000u : 0u;
        v[e] &= (lo | hi);
    }
    return v;
}

__device__ __forceinline__ u32x4 keep_first_f32(u32x4 v, int n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < n ? v[e] : 0u;
    return v;
}

__device__ __forceinline__ u32x4 ldg_nt(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

constexpr u32x4 kZero4 = {0u, 0u, 0u, 0u};

// Exclusive prefix sum of one value per thread over a workgroup of NW waves;
// *total receives the sum.  Every thread must call it.
template <int NW>
__device__ __forceinline__ int block_exscan(int v, int* s_tmp, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = s_tmp[i];
        before += i < w ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// Last index s in [0, n) with cum[s] <= x, for a non-decreasing cum[0..n] with
// cum[0] <= x < cum[n]: the sequence whose items contain item x.
__device__ __forceinline__ int find_seq(const int* cum, int n, int x) {
    int lo = 0, hi = n;                 // cum[lo] <= x < cum[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Per-lane registers of one 32-token chunk.
template <bool BF16, int D>
struct ChunkRegs {
    // K: 2 tiles of 16 rows; per lane D*esize/64 bytes of a row per tile.
    static constexpr int KV = BF16 ? D / 32 : D / 16;    // uint4 per tile
    // V: D/16 channel tiles; per lane 8 tokens of one channel.
    static constexpr int VV = BF16 ? D / 16 : D / 8;     // uint4 per chunk
    u32x4 k[2][KV];
    u32x4 v[VV];
};

// fp32 caches at head_dim 128 hold twice the registers per chunk and run at
// two waves per SIMD; every other variant at three.
template <bool BF16, int D, bool FIXED, bool APPEND>
__global__ __launch_bounds__((64 * waves_per_group<BF16, D, FIXED>()))
__attribute__((amdgpu_waves_per_eu((waves_per_simd<BF16, D>())))) void decode_partition_kernel(DecodeArgs a) {
    constexpr int NW = waves_per_group<BF16, D, FIXED>();   // waves per workgroup
    constexpr int NT = 64 * NW;
    constexpr int WIN = 4 * NW;                              // chunks per window
    constexpr int WINB = WIN * kChunk / kMinBlock + 1;       // block ids a window can touch
    constexpr int SPT = (kMaxSeqsPerLaunch + NT - 1) / NT;   // lengths scanned per thread
    constexpr int HG = FIXED ? 16 : kMergeHeads;             // heads per merge pass
    constexpr int ES = BF16 ? 2 : 4;
    using Regs = ChunkRegs<BF16, D>;
    constexpr int MT = D / 16;                    // output channel tiles
    constexpr int QV = BF16 ? D / 32 : D / 16;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int r = lane & 15;
    const int j = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.G;
    const int H = a.H;
    const int B = a.B;
    const int bs = a.bs;
    const float kNaN = __builtin_nanf("");

    // ---- LDS: (balanced split) lengths and their prefix sums; wave-merge buffers ----
    extern __shared__ int s_dyn[];
    int* s_len = s_dyn;                           // [B]  L, or -1 for an invalid length
    int* s_cum = s_len + B;                       // [B+1] chunks per head before sequence s
    float* s_acc = reinterpret_cast<float*>(FIXED ? s_dyn : s_cum + B + 1);   // [NW][min(G, HG)][D+4]
    __shared__ int s_blk[2][WINB];
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ int s_tmp[NW];

    const int64_t tile_elems = static_cast<int64_t>(H) * bs * D;   // one block, all heads
    int buf = 0;                                                    // s_blk buffer in use

    // Decode with append: store the newest token (position L - 1) of (sequence
    // s, kv head g) at slot new_slots[s] of the pools, one channel per thread
    // (D <= NT).  Slots outside the pool store nothing.
    auto store_newest = [&](int s, int g) {
        if (tid >= D) return;
        const int64_t slot = a.new_slots[s];
        if (slot < 0 || slot >= static_cast<int64_t>(a.N) * bs) return;
        const int64_t src = (static_cast<int64_t>(s) * H + g) * D + tid;
        const int64_t blk = slot / bs, off = slot % bs;
        const int d = tid;
        const int64_t kidx = (blk * H + g) * bs * D + ((d >> 5) * bs + off) * 32 + (d & 31);
        const int64_t vidx = ((blk * H + g) * D + d) * bs + off;
        if constexpr (BF16) {
            static_cast<uint16_t*>(a.kw)[kidx] = static_cast<const uint16_t*>(a.k_new)[src];
            static_cast<uint16_t*>(a.vw)[vidx] = static_cast<const uint16_t*>(a.v_new)[src];
        } else {
            static_cast<uint32_t*>(a.kw)[kidx] = static_cast<const uint32_t*>(a.k_new)[src];
            static_cast<uint32_t*>(a.vw)[vidx] = static_cast<const uint32_t*>(a.v_new)[src];
        }
    };
    // Set once this workgroup has stored newest tokens that it reads back: the
    // next window barrier then carries a workgroup-scope release before it and
    // an acquire after it, which make the stores visible to the workgroup's
    // loads.  Fencing at that barrier rather than right after the stores lets
    // the window's block-id loads overlap the wait for the stores.
    bool fence_pending = false;

    // Balanced split: merged piece results wait in LDS, up to kPendSlots
    // pieces (kPendFloats floats in all), and go to memory when the buffer is
    // full and at the end of the workgroup's range.  Stores issued between
    // pieces hold up the next piece's block-id wait until they are
    // acknowledged, and under a saturating read stream that takes longer than
    // the loads.  Each thread writes and later stores the same entries, and
    // each wave keeps its own copy of the pieces' descriptions, so the buffer
    // needs no barrier.  24 KB keeps three workgroups per CU (static and
    // dynamic LDS stay under 53 KB for 1,024 sequences at head_dim 128).
    __shared__ float s_pend[FIXED ? 1 : kPendFloats];      // [slot][G][D] outputs or partial sums
    __shared__ float2 s_pml[FIXED ? 1 : kPendFloats / D];   // [slot][G] (max, sum) of partial pieces
    __shared__ int s_pmeta[FIXED ? 1 : NW][kPendSlots][3];  // per wave: pieces, piece, first row
    const int pend_cap = FIXED ? 0 : min(kPendSlots, kPendFloats / (G * D));
    int npend = 0;
    auto flush = [&]() {
        for (int p = 0; p < npend; ++p) {
            const int np = s_pmeta[w][p][0], piece = s_pmeta[w][p][1];
            const int64_t sh0 = s_pmeta[w][p][2];
            const float* src = s_pend + p * G * D;
            for (int h0 = 0; h0 < G; h0 += HG) {
                const int hn = min(HG, G - h0);
                for (int e = tid; e < hn * D; e += NT) {
                    const int d = e % D, h = h0 + e / D;
                    const int64_t sh = sh0 + h;
                    const float v = src[h * D + d];
                    if (np == 1) {
                        store_out(a.out, sh * D + d, v, a.out_bf16);
                    } else {
                        a.ws_acc[(sh * a.pmax + piece) * D + d] = v;
                        if (d == 0) a.ws_ml[sh * a.pmax + piece] = s_pml[p * G + h];
                    }
                    if (piece == 0 && d == 0 && a.ws_np) a.ws_np[sh] = np;
                }
            }
        }
        npend = 0;
    };

    // One partition: chunks [cb, ce) of (sequence s, kv head g), the piece-th
    // of its npieces partitions.
    auto process = [&](int s, int g, int L, int cb, int ce, int piece, int npieces) {
        const char* kbase = static_cast<const char*>(a.kc) + static_cast<int64_t>(g) * bs * D * ES;
        const char* vbase = static_cast<const char*>(a.vc) + static_cast<int64_t>(g) * D * bs * ES;
        const int nblk_seq = (L + bs - 1) / bs;
        const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.maxb;
        // Fixed partitions: the piece that holds the newest token stores it
        // first and then reads it back like every other token.  (The balanced
        // split stores all of a workgroup's newest tokens before its first
        // piece.)
        if constexpr (APPEND && FIXED) {
            if (ce > (L - 1) / kChunk) {
                store_newest(s, g);
                fence_pending = true;
            }
        }

        // Query operand: lane (j, r) holds head r's channels for k-group j.
        u32x4 qreg[QV];
        {
            const char* qrow = static_cast<const char*>(a.q) +
                               ((static_cast<int64_t>(s) * a.Hq + g * G + r) * D) * ES;
#pragma unroll
            for (int c = 0; c < QV; ++c) {
                // bf16: channels c*32 + j*8 .. +8;  fp32: channels j*(D/4) + 4c .. +4
                const int d0 = BF16 ? c * 32 + j * 8 : j * (D / 4) + 4 * c;
                qreg[c] = r < G ? *reinterpret_cast<const u32x4*>(qrow + static_cast<int64_t>(d0) * ES)
                                : kZero4;
            }
        }

        float m_run = -INFINITY;
        float l_run = 0.f;
        f32x4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Loads are unconditional: every address is inside the pool (ids of
        // blocks past the sequence's end were replaced by block 0), so no load
        // sits behind a divergent branch and all of a chunk's loads issue back
        // to back.  Rows past the context end are dealt with when the chunk is
        // consumed: their logits are selected to -inf and their values to 0.
        auto load_chunk = [&](int ci, int fb, const int* blk_ids, Regs& R) {
            const int tc = ci * kChunk;               // absolute position of the chunk
            // K: row r of tile t is chunk token 8*(r>>2) + (r&3) + 4t.
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int tp = tc + 8 * (r >> 2) + (r & 3) + 4 * t;
                const int64_t blk = blk_ids[tp / bs - fb];
                const char* tile = kbase + blk * tile_elems * ES;
#pragma unroll
                for (int c = 0; c < Regs::KV; ++c) {
                    // channel d0 of token tp: group d0 / 32, row tp % bs of the group
                    const int d0 = BF16 ? c * 32 + j * 8 : j * (D / 4) + 4 * c;
                    const int64_t e = (static_cast<int64_t>(d0 >> 5) * bs + tp % bs) * 32 + (d0 & 31);
                    R.k[t][c] = ldg_nt(tile + e * ES);
                }
            }
            // V: lane (j, r) reads tokens 8j..8j+7 of channel mt*16 + r.
            const int tp0 = tc + 8 * j;
            const int64_t blk = blk_ids[tp0 / bs - fb];
            const char* vb = vbase + (blk * tile_elems + tp0 % bs) * ES;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int64_t ch = mt * 16 + r;
                if (BF16) {
                    R.v[mt] = ldg_nt(vb + ch * bs * ES);
                } else {
                    R.v[2 * mt] = ldg_nt(vb + ch * bs * ES);
                    R.v[2 * mt + 1] = ldg_nt(vb + ch * bs * ES + 16);
                }
            }
        };

        auto compute_chunk = [&](int ci, const Regs& R) {
            const int tc = ci * kChunk;
            // ---- logits: S^T[token][head] for the chunk's two 16-row tiles ----
            f32x4_t st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BF16) {
#pragma unroll
                    for (int c = 0; c < Regs::KV; ++c)
                        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[t][c]), as_bf16x8(qreg[c]),
                                                                     c4, 0, 0, 0);
                } else {
#pragma unroll
                    for (int c = 0; c < Regs::KV; ++c) {
                        const u32x4 kk = R.k[t][c], qq = qreg[c];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            c4 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kk[e]),
                                                                      __uint_as_float(qq[e]), c4, 0, 0, 0);
                    }
                }
                st[t] = c4;
            }
            // lane (j, r): head r, chunk tokens 8j + e with e = 4t + i
            float sv[8];
            const int ntok = L - (tc + 8 * j);                // valid tokens among this lane's 8
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = st[e >> 2][e & 3] * a.scale_log2;
                sv[e] = e < ntok ? x : -INFINITY;
            }
            float cm = sv[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) cm = fmaxf(cm, sv[e]);
            cm = fmaxf(cm, __shfl_xor(cm, 16));
            cm = fmaxf(cm, __shfl_xor(cm, 32));
            // every chunk of a partition holds at least one valid token, so cm is finite
            const float m_new = fmaxf(m_run, cm);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            float pv[8];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
                psum += pv[e];
            }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
            // ---- values: O^T[channel][head] += V^T[channel][token] . P^T ----
            // A weight of 0 does not cancel a NaN value (never-written slots past
            // the context end), so those values are zeroed by select.
            Regs Rm = R;
            if (tc + kChunk > L) {
#pragma unroll
                for (int x = 0; x < Regs::VV; ++x) {
                    if constexpr (BF16)
                        Rm.v[x] = keep_first_bf16(R.v[x], ntok);
                    else
                        Rm.v[x] = keep_first_f32(R.v[x], (x & 1) ? ntok - 4 : ntok);
                }
            }
            if constexpr (BF16) {
                bf16x8_t ph, pl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const __bf16 hi = static_cast<__bf16>(pv[e]);
                    ph[e] = hi;
                    pl[e] = static_cast<__bf16>(pv[e] - static_cast<float>(hi));
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Rm.v[mt]), ph, acc[mt], 0, 0, 0);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Rm.v[mt]), pl, acc[mt], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 v0 = Rm.v[2 * mt], v1 = Rm.v[2 * mt + 1];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(e < 4 ? v0[e] : v1[e - 4]),
                                                                       pv[e], acc[mt], 0, 0, 0);
                }
            }
        };

        // Windows of up to 4 chunks per wave.  The window's block ids go to one of two
        // LDS buffers, so one barrier per window suffices: a buffer is written
        // again only two windows later, after every wave has passed the barrier
        // that follows its last use.  Block ids past the sequence's end are
        // replaced by block 0; an id outside the pool makes the partition NaN and
        // is never dereferenced.

        int bad = 0;
        for (int wb = cb; wb < ce; wb += WIN) {

            const int we = min(ce, wb + WIN);
            const int fb = (wb * kChunk) / bs;
            const int nb = (we * kChunk - 1) / bs - fb + 1;
            int* ids = s_blk[buf];
            if (tid < nb) {
                const int b = fb + tid;
                int id = 0;
                if (b < nblk_seq) {
                    id = trow[b];
                    if (id < 0 || id >= a.N) {
                        bad = 1;
                        id = 0;
                    }
                }
                ids[tid] = id;
            }
            if constexpr (APPEND) {
                if (fence_pending) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            }
            bad = __syncthreads_or(bad);
            if constexpr (APPEND) {
                if (fence_pending) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                fence_pending = false;
            }
            // Latency is hidden by occupancy (three waves per SIMD), not by a
            // register double buffer: holding a second chunk needs ~280
            // registers, which spills even at two waves per SIMD.
            for (int ci = wb + w; ci < we; ci += NW) {
                Regs R;
                load_chunk(ci, fb, ids, R);
                compute_chunk(ci, R);
            }
            buf ^= 1;
        }

        // ---- merge the waves through LDS, HG heads per pass ----
        const int rowstride = D + 4;
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (j == 0) {
            s_m[w][r] = m_run;
            s_l[w][r] = l_tot;
        }
        const int hstride = min(G, HG);           // head rows per wave in s_acc
        for (int h0 = 0; h0 < G; h0 += HG) {
            const int hn = min(HG, G - h0);
            if (h0 > 0) __syncthreads();          // the previous pass has read s_acc
            if (r >= h0 && r < h0 + hn) {
                float* dst = s_acc + (w * hstride + (r - h0)) * rowstride;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[mt * 16 + 4 * j + i] = acc[mt][i];
            }
            __syncthreads();
            for (int e = tid; e < hn * D; e += NT) {
                const int hl = e / D, d = e % D, h = h0 + hl;
                // a wave with no chunk in this piece has m = -inf and contributes 0
                float M = s_m[0][h];
#pragma unroll
                for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, s_m[ww][h]);
                float o = 0.f, l = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    const float f = __builtin_amdgcn_exp2f(s_m[ww][h] - M);
                    o += f * s_acc[(ww * hstride + hl) * rowstride + d];
                    l += f * s_l[ww][h];
                }
                if constexpr (FIXED) {
                    const int64_t sh = static_cast<int64_t>(s) * a.Hq + g * G + h;
                    if (npieces == 1) {
                        store_out(a.out, sh * D + d, bad ? kNaN : o / l, a.out_bf16);
                    } else {
                        a.ws_acc[(sh * a.pmax + piece) * D + d] = bad ? kNaN : o;
                        if (d == 0) a.ws_ml[sh * a.pmax + piece] = bad ? make_float2(kNaN, kNaN) : make_float2(M, l);
                    }
                    if (piece == 0 && d == 0 && a.ws_np) a.ws_np[sh] = npieces;
                } else {
                    s_pend[npend * G * D + h * D + d] = bad ? kNaN : (npieces == 1 ? o / l : o);
                    if (d == 0) s_pml[npend * G + h] = bad ? make_float2(kNaN, kNaN) : make_float2(M, l);
                }
            }
        }
        if constexpr (!FIXED) {
            // every lane writes the same description, so each reads back its own write
            s_pmeta[w][npend][0] = npieces;
            s_pmeta[w][npend][1] = piece;
            s_pmeta[w][npend][2] = s * a.Hq + g * G;
            if (++npend == pend_cap) flush();
        }
    };

    if constexpr (FIXED) {
        // One workgroup per (sequence, kv head, partition), dispatched by the
        // hardware as slots free up; partitions past a sequence's end exit at
        // once.  An invalid length gives NaN for the head group, written by
        // the workgroup of partition 0.
        const int u = xcd_remap(blockIdx.x, gridDim.x);
        const int s = u % B;
        const int p = (u / B) % a.pmax;
        const int g = u / (B * a.pmax);
        const int part_tokens = a.part_chunks * kChunk;
        const int L = a.lens[s];
        if (L < 1 || L > a.max_ctx) {
            if (p == 0) {
                for (int e = tid; e < G * D; e += NT)
                    store_out(a.out, (static_cast<int64_t>(s) * a.Hq + g * G) * D + e, kNaN, a.out_bf16);
                if (a.ws_np && tid < G) a.ws_np[static_cast<int64_t>(s) * a.Hq + g * G + tid] = 0;
            }
            return;
        }
        const int np = (L + part_tokens - 1) / part_tokens;
        if (p >= np) return;
        const int cb = p * a.part_chunks;
        process(s, g, L, cb, min((L + kChunk - 1) / kChunk, cb + a.part_chunks), p, np);
        return;
    }

    // ---- balanced split: scan the lengths ----
    {
        int cnt[SPT];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int s = tid * SPT + i;
            int L = s < B ? a.lens[s] : -1;
            // the host guarantees max_ctx <= maxb * bs, so a valid L needs no
            // other bound to stay inside the block table
            const bool ok = L >= 1 && L <= a.max_ctx;
            if (!ok) L = -1;
            if (s < B) s_len[s] = L;
            cnt[i] = ok ? (L + kChunk - 1) / kChunk + kPieceSlots : 0;   // chunk slots per head
            sum += cnt[i];
        }
        int tot;
        int pre = block_exscan<NW>(sum, s_tmp, &tot);
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int s = tid * SPT + i;
            if (s < B) s_cum[s] = pre;
            pre += cnt[i];
        }
        if (tid == 0) s_cum[B] = tot;
        __syncthreads();
    }

    // invalid lengths: NaN for every head and no piece (workgroup s % grid)
    for (int s = blockIdx.x; s < B; s += gridDim.x) {
        if (s_len[s] >= 0) continue;
        for (int e = tid; e < a.Hq * D; e += NT)
            store_out(a.out, static_cast<int64_t>(s) * a.Hq * D + e, kNaN, a.out_bf16);
        if (a.ws_np)
            for (int h = tid; h < a.Hq; h += NT) a.ws_np[static_cast<int64_t>(s) * a.Hq + h] = 0;
    }

    // Ranges of Cw chunk slots over the (sequence, kv head, slot) space, laid
    // out sequence by sequence and head by head; a (sequence, head) has
    // kPieceSlots slots with no chunk, then its chunks.  The workgroup index
    // is remapped so that neighbouring ranges run on the same XCD.
    const int64_t T = static_cast<int64_t>(H) * s_cum[B];
    const int64_t grid = gridDim.x;
    const int64_t Cw = max(static_cast<int64_t>(kMinPieceChunks), (T + grid - 1) / grid);
    const int64_t wr = xcd_remap(blockIdx.x, gridDim.x);
    int64_t pos = wr * Cw;
    const int64_t end = min(T, pos + Cw);
    if (pos >= end) return;
    int s = find_seq(s_cum, B, static_cast<int>(pos / H));
    if constexpr (APPEND) {
        // The range holds the last chunk of every (sequence, head) it ends
        // inside (the last slot is always a chunk): store those newest tokens
        // before the first piece, outside the
        // piece loop, so that loop keeps the plain kernel's registers.
        int64_t p2 = pos;
        int s2 = s;
        while (p2 < end) {
            const int n = s_cum[s2 + 1] - s_cum[s2];
            const int64_t base = static_cast<int64_t>(H) * s_cum[s2];
            const int g = static_cast<int>((p2 - base) / n);
            const int off = static_cast<int>((p2 - base) % n);
            const int take = static_cast<int>(min(static_cast<int64_t>(n - off), end - p2));
            if (off + take == n) store_newest(s2, g);
            p2 += take;
            while (s2 < B && p2 >= static_cast<int64_t>(H) * s_cum[s2 + 1]) ++s2;
        }
        fence_pending = true;
    }
    while (pos < end) {
        const int n = s_cum[s + 1] - s_cum[s];          // slots per head of sequence s
        const int64_t base = static_cast<int64_t>(H) * s_cum[s];
        const int g = static_cast<int>((pos - base) / n);
        const int off = static_cast<int>((pos - base) % n);
        const int take = static_cast<int>(min(static_cast<int64_t>(n - off), end - pos));
        const int64_t start_sg = base + static_cast<int64_t>(g) * n;
        // chunks [c0, c1) of the (sequence, head) fall in this range; pieces
        // are the ranges that hold any of its chunks
        const int c0 = max(off, kPieceSlots) - kPieceSlots, c1 = off + take - kPieceSlots;
        if (c1 > c0) {
            const int64_t first = (start_sg + kPieceSlots) / Cw;
            const int64_t last = (start_sg + n - 1) / Cw;
            process(s, g, s_len[s], c0, c1, static_cast<int>(wr - first), static_cast<int>(last - first + 1));
        }
        pos += take;
        while (s < B && pos >= static_cast<int64_t>(H) * s_cum[s + 1]) ++s;
    }
    flush();
}

// Merge the pieces of every (sequence, query head) that has more than one: one
// wave per (sequence, head), four per workgroup.  With M the largest piece max,
// each piece's sum and output are weighted by 2^(m_p - M); the result is their
// ratio.  Lane i owns channels i, i + 64 (D = 128) or i (D = 64); the pieces
// are summed in a fixed order, so the result does not depend on timing.
constexpr int kReduceWaves = 4;
constexpr int kReduceAheadPairs = 4096; // balanced split: (sequence, head) pairs up to which the reduce loads ahead
constexpr int kReduceWgPieces = 16;     // fixed partitions allowing this many pieces per head or more: a workgroup per head

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// KPRE partial rows (and, with MLPRE, the first 64 (max, sum) pairs) are
// loaded together with the piece count, before it is known, so a head with few
// pieces costs one round trip to memory.  That pays where most heads have
// several pieces (fixed partitions of long contexts); under the balanced split
// most heads are a single piece, whose speculative loads are wasted bytes, so
// the host takes fewer there.  All speculative slots lie inside the workspace;
// the ones past the count hold leftovers and are never used (selected away,
// not multiplied by zero, as they may be NaN).
template <int D, int KPRE, bool MLPRE>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(void* out, int out_bf16,
                                                                         const float* __restrict__ ws_acc,
                                                                         const float2* __restrict__ ws_ml,
                                                                         const int32_t* __restrict__ ws_np,
                                                                         int64_t pairs, int32_t P) {
    constexpr int CPL = D / 64;                   // channels per lane
    constexpr int kPre = KPRE;                    // partial rows loaded before the piece count
    const int lane = threadIdx.x & 63;
    const int64_t pair = static_cast<int64_t>(blockIdx.x) * kReduceWaves + (threadIdx.x >> 6);
    if (pair >= pairs) return;
    const int np_raw = ws_np[pair];
    const float2* ml = ws_ml + pair * P;
    float2 ml0 = make_float2(-INFINITY, 0.f);
    if constexpr (MLPRE) ml0 = lane < P ? ml[lane] : ml0;
    const float* accp = ws_acc + pair * P * D + lane;
    float pre[kPre > 0 ? kPre : 1][CPL];
#pragma unroll
    for (int u = 0; u < kPre; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) pre[u][c] = u < P ? accp[static_cast<int64_t>(u) * D + 64 * c] : 0.f;
    const int np = min(np_raw, P);
    if (np <= 1) return;                          // final already, or NaN written
    if constexpr (!MLPRE) ml0 = lane < np ? ml[lane] : ml0;
    float m = lane < np ? ml0.x : -INFINITY;
    for (int i = lane + 64; i < np; i += 64) m = fmaxf(m, ml[i].x);
    const float M = wave_max(m);
    float dp = lane < np ? __builtin_amdgcn_exp2f(ml0.x - M) * ml0.y : 0.f;
    for (int i = lane + 64; i < np; i += 64) {
        const float2 v = ml[i];
        dp += __builtin_amdgcn_exp2f(v.x - M) * v.y;
    }
    const float den = wave_sum(dp);
    // Each lane computes the weight of one piece of a block of 64; the weights
    // are broadcast with shuffles and the channel sums are kept in four
    // independent accumulators, so four loads per lane are in flight.
    float o[4][CPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[u][c] = 0.f;
    for (int b0 = 0; b0 < np; b0 += 64) {
        const int nb = min(64, np - b0);
        const float fl = lane < nb ? __builtin_amdgcn_exp2f((b0 == 0 ? ml0.x : ml[b0 + lane].x) - M) : 0.f;
        int k = 0;
        if (b0 == 0) {
#pragma unroll
            for (int u = 0; u < kPre; ++u) {
                const float f = __shfl(fl, u);
#pragma unroll
                for (int c = 0; c < CPL; ++c) o[u][c] += u < nb ? f * pre[u][c] : 0.f;
            }
            k = kPre;
        }
        for (; k + 4 <= nb; k += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = __shfl(fl, k + u);
                const float* src = accp + static_cast<int64_t>(b0 + k + u) * D;
#pragma unroll
                for (int c = 0; c < CPL; ++c) o[u][c] += f * src[64 * c];
            }
        }
        for (; k < nb; ++k) {
            const float f = __shfl(fl, k);
            const float* src = accp + static_cast<int64_t>(b0 + k) * D;
#pragma unroll
            for (int c = 0; c < CPL; ++c) o[0][c] += f * src[64 * c];
        }
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float v = ((o[0][c] + o[1][c]) + (o[2][c] + o[3][c])) * inv;
        const int64_t idx = pair * D + lane + 64 * c;
        if (out_bf16)
            static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);
        else
            static_cast<float*>(out)[idx] = v;
    }
}

// Many pieces per head (fixed partitions of long contexts): one 4-wave
// workgroup per (sequence, query head), so a batch of few long sequences still
// spreads its merge over the chip.  Every wave finds the largest piece max M
// and the denominator over all pieces itself (lanes take pieces, 64 at a
// time); wave w sums the weighted partial rows of pieces w, w + 4, w + 8, ...,
// four rows in flight per lane, and the four sums are added through LDS in
// wave order, so the result does not depend on timing.
template <int D>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_wg_kernel(void* out, int out_bf16,
                                                                            const float* __restrict__ ws_acc,
                                                                            const float2* __restrict__ ws_ml,
                                                                            const int32_t* __restrict__ ws_np,
                                                                            int64_t pairs, int32_t P) {
    constexpr int CPL = D / 64;                   // channels per lane
    constexpr int NW = kReduceWaves;
    __shared__ float s_o[NW][D];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t pair = blockIdx.x;
    if (pair >= pairs) return;
    const int np = min(ws_np[pair], P);
    if (np <= 1) return;                          // final already, or NaN written (the whole workgroup)
    const float2* ml = ws_ml + pair * P;
    float m = -INFINITY;
    for (int i = lane; i < np; i += 64) m = fmaxf(m, ml[i].x);
    const float M = wave_max(m);
    float dp = 0.f;
    for (int i = lane; i < np; i += 64) {
        const float2 v = ml[i];
        dp += __builtin_amdgcn_exp2f(v.x - M) * v.y;
    }
    const float den = wave_sum(dp);
    const float* accp = ws_acc + pair * P * D + lane;
    float o[4][CPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[u][c] = 0.f;
    for (int b0 = 0; b0 < np; b0 += 64) {
        const int nb = min(64, np - b0);
        const float fl = lane < nb ? __builtin_amdgcn_exp2f(ml[b0 + lane].x - M) : 0.f;
        int k = w;
        for (; k + 3 * NW < nb; k += 4 * NW) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = __shfl(fl, k + u * NW);
                const float* src = accp + static_cast<int64_t>(b0 + k + u * NW) * D;
#pragma unroll
                for (int c = 0; c < CPL; ++c) o[u][c] += f * src[64 * c];
            }
        }
        for (; k < nb; k += NW) {
            const float f = __shfl(fl, k);
            const float* src = accp + static_cast<int64_t>(b0 + k) * D;
#pragma unroll
            for (int c = 0; c < CPL; ++c) o[0][c] += f * src[64 * c];
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) s_o[w][lane + 64 * c] = (o[0][c] + o[1][c]) + (o[2][c] + o[3][c]);
    __syncthreads();
    if (w != 0) return;
    const float inv = 1.f / den;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int i = lane + 64 * c;
        const float v = ((s_o[0][i] + s_o[1][i]) + (s_o[2][i] + s_o[3][i])) * inv;
        const int64_t idx = pair * D + i;
        if (out_bf16)
            static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);
        else
            static_cast<float*>(out)[idx] = v;
    }
}

// ---- host side ----------------------------------------------------------------------
struct Plan {
    int32_t part_chunks;   // 0 = balanced
    int32_t pmax;          // piece slots per (sequence, head); <= 1 means no workspace
    int32_t G;
};

// Piece slots per (sequence, head): fixed partitions need ceil(max_ctx / P);
// balanced ranges of >= kMinPieceChunks chunk slots cut a head's n chunks (n
// consecutive slots) into at most ceil(n / kMinPieceChunks) + 1 pieces.
int32_t piece_slots(int32_t max_context_len, int32_t part_chunks) {
    const int64_t nch = (static_cast<int64_t>(max_context_len) + kChunk - 1) / kChunk;
    if (part_chunks > 0) return static_cast<int32_t>((nch + part_chunks - 1) / part_chunks);
    return static_cast<int32_t>((nch + kMinPieceChunks - 1) / kMinPieceChunks + 1);
}

int plan_partition(int32_t partition_size, int32_t* part_chunks) {
    if (partition_size == 0) {
        *part_chunks = 0;
        return PA_OK;
    }
    if (partition_size < kChunk || partition_size % kChunk || partition_size > (1 << 20))
        return PA_ERR_UNSUPPORTED;
    *part_chunks = partition_size / kChunk;
    return PA_OK;
}

int check_decode(const pa_cache_desc* desc, int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads,
                 int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                 Plan* c) {
    if (!desc_ok(desc) || num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 ||
        max_context_len < 1)
        return PA_ERR_INVALID_ARG;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    const int32_t H = desc->num_kv_heads;
    if (num_q_heads % H) return PA_ERR_INVALID_ARG;
    const int32_t G = num_q_heads / H;
    int rc = plan_partition(partition_size, &c->part_chunks);
    if (rc != PA_OK) return rc;
    const int32_t bs = desc->block_size;
    if (!is_pow2(bs) || bs < kMinBlock || bs > 256) return PA_ERR_UNSUPPORTED;
    if (G > 16) return PA_ERR_UNSUPPORTED;
    if (desc->head_dim != 64 && desc->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * bs)
        return PA_ERR_INVALID_ARG;
    c->pmax = piece_slots(max_context_len, c->part_chunks);
    c->G = G;
    return PA_OK;
}

// Workspace: the partials [B][Hq][pmax][D], their (max, sum) pairs
// [B][Hq][pmax] and the piece count of every (sequence, head) [B][Hq].  None
// is needed when every context fits one fixed partition.
struct WsLayout {
    size_t acc, ml, np, total;   // byte offsets of the three arrays and the total size
};

WsLayout workspace_layout(int64_t B, int64_t Hq, int64_t D, int64_t pmax, bool fixed) {
    WsLayout l{0, 0, 0, 0};
    if (fixed && pmax <= 1) return l;
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    l.acc = 0;
    l.ml = static_cast<size_t>(al(B * Hq * pmax * D * 4));
    l.np = l.ml + static_cast<size_t>(al(B * Hq * pmax * 8));
    l.total = l.np + static_cast<size_t>(B * Hq * 4);
    return l;
}

size_t decode_lds_bytes(int32_t nseq, int32_t G, int32_t D, bool fixed, int waves) {
    const int heads = fixed ? G : std::min(G, kMergeHeads);
    return (fixed ? 0 : static_cast<size_t>(2 * nseq + 1) * sizeof(int)) +
           static_cast<size_t>(waves) * heads * (D + 4) * sizeof(float);
}

// Compute units of the current device (cached per device).
int device_cus(int* cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    int rc = hip_status(hipGetDevice(&dev));
    if (rc != PA_OK) return rc;
    if (dev >= 0 && dev < 64) {
        const int n = cache[dev].load(std::memory_order_relaxed);
        if (n > 0) {
            *cus = n;
            return PA_OK;
        }
    }
    int n = 0;
    rc = hip_status(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
    if (rc != PA_OK) return rc;
    if (n <= 0) return PA_ERR_HIP;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return PA_OK;
}

// Events set by pa_time_next_partitions for the next partition pass of this
// host thread: start goes with its first kernel launch, stop with its last.
struct PartitionTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
thread_local PartitionTiming g_time_next;

template <bool BF16, int D>
int launch_partitions(const DecodeArgs& a0, int32_t num_seqs, const Plan& c, hipStream_t st) {
    const PartitionTiming timing = g_time_next;
    g_time_next = PartitionTiming{};
    const bool fixed = c.part_chunks > 0;
    const bool app = a0.k_new != nullptr;
    const auto kernel = fixed ? (app ? decode_partition_kernel<BF16, D, true, true>
                                     : decode_partition_kernel<BF16, D, true, false>)
                              : (app ? decode_partition_kernel<BF16, D, false, true>
                                     : decode_partition_kernel<BF16, D, false, false>);
    const int waves = fixed ? waves_per_group<BF16, D, true>() : waves_per_group<BF16, D, false>();
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != PA_OK) return rc;
    constexpr int ES = BF16 ? 2 : 4;
    const size_t per_seq_acc = static_cast<size_t>(a0.Hq) * c.pmax * D * 4;
    const size_t per_seq_ml = static_cast<size_t>(a0.Hq) * c.pmax * 8;
    for (int32_t s0 = 0; s0 < num_seqs; s0 += kMaxSeqsPerLaunch) {
        const int32_t nb = std::min(kMaxSeqsPerLaunch, num_seqs - s0);
        DecodeArgs a = a0;
        a.B = nb;
        a.out = static_cast<char*>(a0.out) + static_cast<int64_t>(s0) * a0.Hq * D * (a0.out_bf16 ? 2 : 4);
        a.q = static_cast<const char*>(a0.q) + static_cast<int64_t>(s0) * a0.Hq * D * ES;
        a.tables = a0.tables + static_cast<int64_t>(s0) * a0.maxb;
        a.lens = a0.lens + s0;
        if (a0.k_new) {
            a.k_new = static_cast<const char*>(a0.k_new) + static_cast<int64_t>(s0) * a0.H * D * ES;
            a.v_new = static_cast<const char*>(a0.v_new) + static_cast<int64_t>(s0) * a0.H * D * ES;
            a.new_slots = a0.new_slots + s0;
        }
        if (a0.ws_np) {
            a.ws_acc = reinterpret_cast<float*>(reinterpret_cast<char*>(a0.ws_acc) + s0 * per_seq_acc);
            a.ws_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(a0.ws_ml) + s0 * per_seq_ml);
            a.ws_np = a0.ws_np + static_cast<int64_t>(s0) * a0.Hq;
        }
        const size_t lds = decode_lds_bytes(nb, c.G, D, fixed, waves);
        int64_t grid;
        if (fixed) {
            // one workgroup per (sequence, kv head, partition slot)
            grid = static_cast<int64_t>(nb) * a.H * c.pmax;
            if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
        } else {
            // as many workgroups as the chip holds at once, and no more than
            // minimal ranges of the longest context could keep busy
            int per_cu = 0;
            // sized by the plain kernel even for the append variant, so that both
            // cut the batch at the same points and round identically
            rc = hip_status(hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, decode_partition_kernel<BF16, D, false, false>, 64 * waves, lds));
            if (rc != PA_OK) return rc;
            if (per_cu < 1) return PA_ERR_UNSUPPORTED;
            const int64_t nch = (static_cast<int64_t>(a.max_ctx) + kChunk - 1) / kChunk;
            const int64_t items =
                static_cast<int64_t>(nb) * a.H * ((nch + kPieceSlots + kMinPieceChunks - 1) / kMinPieceChunks);
            grid = std::max<int64_t>(1, std::min<int64_t>(static_cast<int64_t>(per_cu) * cus, items));
        }
        rc = launch_kernel_timed(kernel, dim3(static_cast<uint32_t>(grid)), dim3(64 * waves), lds, st,
                                 s0 == 0 ? timing.start : nullptr,
                                 s0 + kMaxSeqsPerLaunch >= num_seqs ? timing.stop : nullptr, a);
        if (rc != PA_OK) return rc;
    }
    return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
    int32_t part_chunks = 0;
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 1 ||
        pa::plan_partition(partition_size, &part_chunks) != PA_OK)
        return 0;
    const int32_t pmax = pa::piece_slots(max_context_len, part_chunks);
    return pa::workspace_layout(num_seqs, num_q_heads, head_dim, pmax, part_chunks > 0).total;
}

}  // extern "C"

namespace pa {
namespace {

// The split-K pass; with k_new non-null, also the append of each sequence's
// newest token (kw/vw are then the writable pools).
int decode_partitions(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                      const void* v_cache, const pa_cache_desc* desc, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t max_context_len, float scale,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream,
                      const void* k_new, const void* v_new, const int64_t* new_slots, void* kw,
                      void* vw) {
    Plan c;
    int rc = check_decode(desc, out_dtype, num_seqs, num_q_heads, max_blocks_per_seq, max_context_len,
                          partition_size, &c);
    if (rc != PA_OK) return rc;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
    // 16-byte loads of q and the pools; element accesses of k_new and v_new
    const uintptr_t esize = desc->kv_dtype == PA_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache)) % 16 ||
        (reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % esize)
        return PA_ERR_INVALID_ARG;
    const int32_t D = desc->head_dim;
    const WsLayout ws = workspace_layout(num_seqs, num_q_heads, D, c.pmax, c.part_chunks > 0);
    if (ws.total > 0 && (!workspace || workspace_bytes < ws.total || reinterpret_cast<uintptr_t>(workspace) % 8))
        return PA_ERR_INVALID_ARG;

    DecodeArgs a;
    a.out = out;
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = context_lens;
    char* wsb = static_cast<char*>(workspace);
    a.ws_acc = ws.total ? reinterpret_cast<float*>(wsb + ws.acc) : nullptr;
    a.ws_ml = ws.total ? reinterpret_cast<float2*>(wsb + ws.ml) : nullptr;
    a.ws_np = ws.total ? reinterpret_cast<int32_t*>(wsb + ws.np) : nullptr;
    a.k_new = k_new;
    a.v_new = v_new;
    a.new_slots = new_slots;
    a.kw = kw;
    a.vw = vw;
    a.B = num_seqs;
    a.Hq = num_q_heads;
    a.H = desc->num_kv_heads;
    a.G = c.G;
    a.bs = desc->block_size;
    a.N = desc->num_blocks;
    a.maxb = max_blocks_per_seq;
    a.max_ctx = max_context_len;
    a.part_chunks = c.part_chunks;
    a.pmax = c.pmax;
    a.scale_log2 = scale * kLog2e;
    a.out_bf16 = out_dtype == PA_BF16;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (desc->kv_dtype == PA_BF16)
        return D == 128 ? launch_partitions<true, 128>(a, num_seqs, c, st)
                        : launch_partitions<true, 64>(a, num_seqs, c, st);
    return D == 128 ? launch_partitions<false, 128>(a, num_seqs, c, st)
                    : launch_partitions<false, 64>(a, num_seqs, c, st);
}

}  // namespace
}  // namespace pa

extern "C" {

int pa_decode_partitions(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                         const void* v_cache, const pa_cache_desc* desc,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_context_len, float scale, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return pa::decode_partitions(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                                 max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                 max_context_len, scale, partition_size, workspace, workspace_bytes,
                                 stream, nullptr, nullptr, nullptr, nullptr, nullptr);
}

int pa_decode_append_partitions(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                const void* v_new, const int64_t* slot_mapping, void* k_cache,
                                void* v_cache, const pa_cache_desc* desc,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_context_len, float scale,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
    return pa::decode_partitions(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                                 max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                 max_context_len, scale, partition_size, workspace, workspace_bytes,
                                 stream, k_new, v_new, slot_mapping, k_cache, v_cache);
}

int pa_time_next_partitions(void* start_event, void* stop_event) {
    pa::g_time_next.start = static_cast<hipEvent_t>(start_event);
    pa::g_time_next.stop = static_cast<hipEvent_t>(stop_event);
    return PA_OK;
}

int pa_decode_reduce(void* out, int32_t out_dtype, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace pa;
    (void)context_lens;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 1) return PA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    int32_t part_chunks = 0;
    int rc = plan_partition(partition_size, &part_chunks);
    if (rc != PA_OK) return rc;
    const int32_t pmax = piece_slots(max_context_len, part_chunks);
    const WsLayout ws = workspace_layout(num_seqs, num_q_heads, head_dim, pmax, part_chunks > 0);
    if (ws.total == 0 || num_seqs == 0) return PA_OK;    // every head is a single partition
    if (!out || !workspace || workspace_bytes < ws.total) return PA_ERR_INVALID_ARG;
    const char* wsb = static_cast<const char*>(workspace);
    const int64_t pairs = static_cast<int64_t>(num_seqs) * num_q_heads;
    if (part_chunks > 0 && pmax >= kReduceWgPieces) {
        // heads of up to pmax pieces: a workgroup per (sequence, query head)
        if (pairs > INT32_MAX) return PA_ERR_UNSUPPORTED;
        const auto kernel = head_dim == 128 ? decode_reduce_wg_kernel<128> : decode_reduce_wg_kernel<64>;
        return launch_kernel(kernel, dim3(static_cast<uint32_t>(pairs)), dim3(64 * kReduceWaves), 0,
                             static_cast<hipStream_t>(stream), out, out_dtype == PA_BF16,
                             reinterpret_cast<const float*>(wsb + ws.acc),
                             reinterpret_cast<const float2*>(wsb + ws.ml),
                             reinterpret_cast<const int32_t*>(wsb + ws.np), pairs, pmax);
    }
    const int64_t grid = (pairs + kReduceWaves - 1) / kReduceWaves;
    if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
    // Four rows and the (max, sum) pairs ahead of the count for fixed
    // partitions, and for a balanced split of a small batch (few heads share
    // the ranges, so most are cut into several pieces: one sequence of 512
    // tokens 8.1 us against 16.4 us without).  A balanced split of a large
    // batch leaves most heads whole: nothing ahead of the count (a lognormal
    // batch of 240, caches cold: 11.0 us against 18.8 us, 13.1 us with one row
    // ahead).
    const bool ahead = part_chunks > 0 || pairs <= kReduceAheadPairs;
    const auto kernel = ahead ? (head_dim == 128 ? decode_reduce_kernel<128, 4, true>
                                                 : decode_reduce_kernel<64, 4, true>)
                              : (head_dim == 128 ? decode_reduce_kernel<128, 0, false>
                                                 : decode_reduce_kernel<64, 0, false>);
    return launch_kernel(kernel, dim3(static_cast<uint32_t>(grid)), dim3(64 * kReduceWaves), 0,
                         static_cast<hipStream_t>(stream), out, out_dtype == PA_BF16,
                         reinterpret_cast<const float*>(wsb + ws.acc),
                         reinterpret_cast<const float2*>(wsb + ws.ml),
                         reinterpret_cast<const int32_t*>(wsb + ws.np), pairs, pmax);
}

int pa_decode_append(void* out, int32_t out_dtype, const void* q, const void* k_new, const void* v_new,
                     const int64_t* slot_mapping, void* k_cache, void* v_cache, const pa_cache_desc* desc,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len, float scale,
                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = pa_decode_append_partitions(out, out_dtype, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                         desc, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                         num_q_heads, max_context_len, scale, partition_size, workspace,
                                         workspace_bytes, stream);
    if (rc != PA_OK) return rc;
    return pa_decode_reduce(out, out_dtype, context_lens, num_seqs, num_q_heads,
                            desc ? desc->head_dim : 0, max_context_len, partition_size, workspace,
                            workspace_bytes, stream);
}

int pa_decode(void* out, int32_t out_dtype, const void* q, const void* k_cache, const void* v_cache,
              const pa_cache_desc* desc, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
              size_t workspace_bytes, void* stream) {
    int rc = pa_decode_partitions(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                  max_context_len, scale, partition_size, workspace, workspace_bytes,
                                  stream);
    if (rc != PA_OK) return rc;
    return pa_decode_reduce(out, out_dtype, context_lens, num_seqs, num_q_heads,
                            desc ? desc->head_dim : 0, max_context_len, partition_size, workspace,
                            workspace_bytes, stream);
}

}  // extern "C"

// ---- decode without allocation --------------------------------------------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc): pa_decode with the
// workspace in this fixed array instead of caller memory.  Every device the
// library runs on holds its own copy for the life of the process.  In host
// code the array's name is only a stand-in: its device address, looked up once
// per device, is what the kernels are given.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_NO_ALLOC_MAX_WORKSPACE];

namespace pa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call for each device).
int scratch_address(void** out) {
    int dev = 0;
    int rc = hip_status(hipGetDevice(&dev));
    if (rc != PA_OK) return rc;
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
            if (rc != PA_OK) return rc;
            if (!p) return PA_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" int pa_decode_no_alloc(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                  const void* v_cache, const pa_cache_desc* desc,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, float scale, int32_t partition_size,
                                  void* stream) {
    // argument checks of pa_decode first (no device is touched for a bad call)
    pa::Plan c;
    int rc = pa::check_decode(desc, out_dtype, num_seqs, num_q_heads, max_blocks_per_seq,
                              max_context_len, partition_size, &c);
    if (rc != PA_OK) return rc;
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, desc->head_dim,
                                                  max_context_len, partition_size);
    if (need > PA_DECODE_NO_ALLOC_MAX_WORKSPACE) return PA_ERR_TOO_LARGE;
    if (num_seqs == 0) return PA_OK;
    void* ws = nullptr;
    if (need > 0) {
        rc = pa::scratch_address(&ws);
        if (rc != PA_OK) return rc;
    }
    return pa_decode(out, out_dtype, q, k_cache, v_cache, desc, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, num_q_heads, max_context_len, scale, partition_size, ws,
                     need, stream);
}
