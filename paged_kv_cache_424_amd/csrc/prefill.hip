// Causal attention of prefill chunks over their paged context (gfx950, bf16).
//
// The prefill half of a continuous-batching step: new requests' prompt chunks
// run in the same step as other requests' decode tokens ([studynote 223] "KV
// Cache PagedAttention", section IV checklist item 2; [studynote 528] "vLLM
// PagedAttention KV cache optimization", section II continuous-batching
// table).  A chunk of C queries is the last C positions of a context of L
// tokens that is already in the paged cache; query i (position L - C + i) sees
// positions 0 .. L - C + i.
//
// Work decomposition.  One workgroup (4 waves) per (chunk, kv head, tile of
// 128 rows), a row being one (query position, query head of the kv head's
// group): 128/G positions x G heads.  The (chunk, head) pairs are spread over
// the eight XCDs and taken longest first (see the kernel's prologue).  Each
// wave owns 32 rows -- one 32-row column of a 32x32 MFMA tile -- and keeps
// their query fragments in registers for the whole walk.  The workgroup walks the key positions in tiles of 64.
// Each tile's K rows and V channel rows are copied from their physical blocks
// into LDS one tile ahead (the loads for tile t+1 are in flight while tile t
// is consumed, double-buffered LDS, one barrier per tile), and the block ids
// two tiles ahead, so no table lookup sits on the critical path.  Two
// workgroups share a CU and their barriers are independent, so one's softmax
// overlaps the other's matrix work.
//
// Matrix cores: S^T[key][row] = K . Q^T and O^T[channel][row] += V^T . P^T with
// v_mfma_f32_32x32x16_bf16.  In a 32x32 output a lane holds 16 rows of one
// column, so a lane owns one query row: its softmax statistics need one
// cross-lane step (the two halves of the wave), and its rescale and final
// normalisation are lane-local.  The K rows of each 32-key MFMA tile are read
// in a permuted order so that the logits a lane receives are exactly the
// weights it must supply, as the value MFMA's B operand, for keys
// 16 kb + 8 h .. +7 (h = lane / 32).  Weights enter the value MFMA as bf16
// (8-bit mantissa, fp32 accumulation).  The running maximum is raised lazily:
// only when a tile's maximum exceeds it by more than 2^8 in weight, so the
// accumulator is rescaled a few times per row rather than per tile; weights
// stay below 2^8, exact in the fp32 sums.  The LDS tiles are XOR-swizzled
// (see the kernel's shared arrays) so that each quarter-wave's 16-byte reads
// hit 16 different bank groups.

#include <cmath>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;        // 128 rows per workgroup
constexpr int kKT = 64;                   // keys per tile
constexpr int kD = 128;
constexpr int kKS = kD / 16;              // k-steps of the logits MFMA (16 channels each)
constexpr int kMT = kD / 32;              // 32-channel tiles of the output
constexpr int kKB = kKT / 16;             // 16-key blocks of the value MFMA
constexpr int kMinBlock = 8;
constexpr float kLazyLog2 = 8.f;          // raise the running max only when it grows by > 2^8
constexpr int kMaxSortedChunks = 256;     // chunks ranked by length inside the kernel

struct PrefillArgs {
    void* out;
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* tables;
    const int32_t* lens;
    const int32_t* qsl;
    int32_t num_chunks, Hq, H, G, log2G, bs, log2bs, N, maxb, max_q, nqt, total_q;
    float scale_log2;
    int32_t out_bf16;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4 keep_first_bf16(u32x4 v, int n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (2 * e < n) ? 0x0000ffffu : 0u;
        const uint32_t hi = (2 * e + 1 < n) ? 0xffff0000u : 0u;
        v[e] &= (lo | hi);
    }
    return v;
}

constexpr u32x4 kZero4 = {0u, 0u, 0u, 0u};

// 16 bytes per lane from global memory straight into LDS: lane i's bytes go
// to dst + 16 i (dst is the same for the whole wave, passed in m0).  Written
// as inline assembly on purpose: the compiler's form of this load makes it
// wait for the load before the next LDS read of any buffer, which would
// serialise the prefetch of tile t + 1 with the math of tile t.  The caller
// waits for vmcnt to reach zero and then for a barrier before the data is
// read.  m0v is the LDS byte address of the wave's destination.
// load_to_lds takes a 64-bit address per lane; load_to_lds_s a scalar 64-bit
// base plus a 32-bit offset per lane.
__device__ __forceinline__ void load_to_lds(const char* src, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0v) : "memory", "m0");
}
__device__ __forceinline__ void load_to_lds_s(const char* sbase, uint32_t voff, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}
// LDS byte address of a shared-memory location (the same for every lane)
__device__ __forceinline__ uint32_t lds_address(const uint16_t* p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)p)));
}
constexpr bf16x2_t kOnes2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

// x of lane (l + 32) mod 64: one lane swap between the wave's halves.  After
// v_permlane32_swap of (x, x) the first result holds the low half's values in
// both halves and the second the high half's.
__device__ __forceinline__ float other_half(float x) {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const int lane = threadIdx.x & 63;
    return __uint_as_float(lane < 32 ? pr[1] : pr[0]);
}

// Key (within a 32-key MFMA tile) whose K row feeds A-operand row r: rows
// r = 8j + 4h + i take key 16 (j / 2) + 8 h + 4 (j % 2) + i, so that output
// element e of lane (h = lane / 32) holds key 16 (e / 8) + 8 h + e % 8.
__device__ __forceinline__ int k_row_key(int r) {
    const int j = r >> 3, h = (r >> 2) & 1, i = r & 3;
    return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + i;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    PrefillArgs a) {
    // K tile [key][channel], rows of 256 bytes: 16-byte segment s of row r
    // sits at position s ^ (r & 15).  V tile [channel][key], rows of 128
    // bytes: segment s of row d sits at position s ^ ((d >> 1) & 7).  The
    // swizzles put the 16 rows a quarter-wave reads at one segment on 16
    // different bank groups.
    __shared__ __align__(16) uint16_t sK[2][kKT * kD];
    __shared__ __align__(16) uint16_t sV[2][kD * kKT];
    __shared__ int s_order[kMaxSortedChunks];
    __shared__ int s_clen[kMaxSortedChunks];       // context length of every chunk
    __shared__ int s_qsl[kMaxSortedChunks + 1];    // query start of every chunk, and the end

    // ---- which (chunk, kv head, query tile) this workgroup takes ----
    // Workgroup b runs on XCD b % 8 (dispatch is round robin over the XCDs).
    // The (chunk, kv head) pairs are dealt round robin to the XCDs, so every
    // XCD gets a share of every chunk while the query tiles of one pair --
    // which read the same K/V -- stay on one XCD and share its L2.  Within
    // an XCD the work goes longest first: chunks by decreasing context
    // length (ranked here from the lengths, when there are few enough
    // chunks), query tiles of a chunk from the last one down.
    const int tid = threadIdx.x;
    const int nc = a.num_chunks;
    const bool few = nc <= kMaxSortedChunks;
    if (few) {
        // every chunk's length and query start read once, in parallel, then
        // ranked from LDS
        for (int i = tid; i <= nc; i += kThreads) {
            if (i < nc) s_clen[i] = a.lens[i];
            s_qsl[i] = a.qsl[i];
        }
        __syncthreads();
        for (int i = tid; i < nc; i += kThreads) {
            const int Li = s_clen[i];
            int rank = 0;
            for (int jc = 0; jc < nc; ++jc) {
                const int Lj = s_clen[jc];
                rank += (Lj > Li) || (Lj == Li && jc < i);
            }
            s_order[rank] = i;
        }
        __syncthreads();
    }
    const int xcd = blockIdx.x % kNumXcds;
    const int k = blockIdx.x / kNumXcds;
    const int npairs = nc * a.H;
    const int npairs_x = (npairs - xcd + kNumXcds - 1) / kNumXcds;   // pairs xcd, xcd + 8, ...
    if (k >= npairs_x * a.nqt) return;
    const int pr = xcd + kNumXcds * (k / a.nqt);                      // pair in longest-first order
    const int qt = a.nqt - 1 - (k % a.nqt);
    const int g = pr % a.H;
    const int c = __builtin_amdgcn_readfirstlane(few ? s_order[pr / a.H] : pr / a.H);
    const int G = a.G;
    const int QT = kRows >> a.log2G;              // query positions per tile

    const int lane = tid & 63;
    const int col = lane & 31;                    // this lane's row within the wave's 32
    const int hh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int qs0 = __builtin_amdgcn_readfirstlane(few ? s_qsl[c] : a.qsl[c]);
    const int Cc = __builtin_amdgcn_readfirstlane(few ? s_qsl[c + 1] : a.qsl[c + 1]) - qs0;
    const int Lc = __builtin_amdgcn_readfirstlane(few ? s_clen[c] : a.lens[c]);
    const bool bad_chunk = qs0 < 0 || Cc < 0 || Cc > a.max_q || qs0 + Cc > a.total_q || Lc < Cc ||
                           static_cast<int64_t>(Lc) > static_cast<int64_t>(a.maxb) * a.bs;
    const float kNaN = __builtin_nanf("");
    if (bad_chunk) {
        // Rows of a malformed chunk cannot be placed safely; if the start and
        // count still address real rows, those rows get NaN.
        if (qs0 >= 0 && Cc > 0 && static_cast<int64_t>(qs0) + Cc <= a.total_q && qt * QT < Cc) {
            for (int e = tid; e < kRows * kD; e += kThreads) {
                const int rho = e / kD, d = e % kD;
                const int qi = qt * QT + (rho >> a.log2G);
                if (qi < Cc) {
                    const int64_t o = (static_cast<int64_t>(qs0 + qi) * a.Hq + g * G + (rho & (G - 1))) * kD + d;
                    if (a.out_bf16) static_cast<__bf16*>(a.out)[o] = static_cast<__bf16>(kNaN);
                    else static_cast<float*>(a.out)[o] = kNaN;
                }
            }
        }
        return;
    }
    if (qt * QT >= Cc) return;
    const int P0 = Lc - Cc;                                    // position of query 0
    const int qhi = min(Cc, (qt + 1) * QT);                    // queries [qt*QT, qhi)
    const int nkt = (P0 + qhi + kKT - 1) / kKT;                // key tiles to visit

    // ---- this lane's row and its query fragments (B operand, k-step ks) ----
    const int rho = 32 * w + col;
    const int qi = qt * QT + (rho >> a.log2G);
    const bool rowok = qi < Cc;
    const int rowpos = P0 + qi;                                // absolute position of the row
    u32x4 qf[kKS];
    {
        const uint16_t* qrow =
            a.q + (static_cast<int64_t>(qs0 + (rowok ? qi : 0)) * a.Hq + g * G + (rho & (G - 1))) * kD;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hh);
            qf[ks] = rowok ? x : kZero4;
        }
    }

    // ---- block ids: tile t touches blocks (64 t) / bs + [0, n_ids) ----
    const int bs = a.bs;
    const int log2bs = a.log2bs;                  // block sizes are powers of two
    const int n_ids = bs >= kKT ? 1 : kKT >> log2bs;
    const int nblk = (Lc + bs - 1) >> log2bs;
    const int32_t* trow = a.tables + static_cast<int64_t>(c) * a.maxb;
    int bad = 0;                                  // the same in every lane
    // The table entry of block i of tile t (clamped to the last block of the
    // context: any valid block, masked later).
    auto block_index = [&](int t, int i) { return ((t * kKT) >> log2bs) + i; };
    auto raw_block_id = [&](int b) { return trow[min(b, nblk - 1)]; };   // nblk >= 1

    // ---- tile loader: global -> LDS directly (no registers), 16 bytes per lane ----
    // Such a load writes its wave's 64 segments to 64 consecutive LDS
    // segments, so the swizzle is applied by choosing which global segment
    // each lane fetches.  K: load p of wave w fills rows 16 w + 4 p .. +3
    // (lane / 16 picks the row, lane % 16 the position); V: load p of wave w
    // fills channel rows 32 w + 8 p .. +7 (lane / 8 the row, lane % 8 the
    // position).  A K segment (8 channels of one key) lies in one 32-channel
    // group of its block, a V segment (8 keys of one channel) in one block,
    // as block_size >= 8.  With block_size <= 64 a tile starts on a block
    // boundary, so each segment's block slot and in-block offset are the same
    // for every tile and are computed once here; larger blocks add the tile's
    // offset inside its block.
    const bool big_blocks = bs > kKT;
    const int64_t tile_bytes = static_cast<int64_t>(a.H) * bs * kD * 2;
    const char* kbase = reinterpret_cast<const char*>(a.kc) + static_cast<int64_t>(g) * bs * kD * 2;
    const char* vbase = reinterpret_cast<const char*>(a.vc) + static_cast<int64_t>(g) * kD * bs * 2;
    int kslot[4];                    // block slot of K load p: the same for the whole wave
    int koff[4], vslot[4], voff[4];  // per lane
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int key = 16 * w + 4 * p + (lane >> 4);
        const int seg = (lane & 15) ^ (key & 15);              // channels 8 seg .. +7
        kslot[p] = big_blocks ? 0 : (16 * w + 4 * p) >> log2bs;
        koff[p] = (((seg >> 2) * bs + (big_blocks ? key : key & (bs - 1))) * 32 + (seg & 3) * 8) * 2;
        const int d = 32 * w + 8 * p + (lane >> 3);
        const int vkey = 8 * ((lane & 7) ^ ((d >> 1) & 7));    // keys vkey .. +7
        vslot[p] = big_blocks ? 0 : vkey >> log2bs;
        voff[p] = (d * bs + (big_blocks ? vkey : vkey & (bs - 1))) * 2;
    }
    // A tile's block ids are read two tiles ahead, lane i taking id i (a
    // vector load, waited for with the tile's own loads; lanes past n_ids
    // repeat the last one), and checked per lane: an id outside the pool
    // marks the workgroup bad and is replaced by block 0, so it is never
    // dereferenced.  A K load instruction reads one block, so its id is
    // taken from its lane into a scalar register and the load's address is
    // that block plus a fixed per-lane offset; a V load instruction spans the
    // tile's blocks, so each lane fetches the id it needs from the lane that
    // holds it.
    auto load_raw = [&](int t) { return raw_block_id(block_index(t, min(lane, n_ids - 1))); };
    auto check_ids = [&](int t, int raw) {
        const int b = block_index(t, min(lane, n_ids - 1));
        const bool inside = b < nblk;
        const bool ok = raw >= 0 && raw < a.N;
        if (__builtin_amdgcn_ballot_w64(inside && !ok)) bad = 1;
        return inside && ok ? raw : 0;
    };
    struct TileIds {
        int k[4];   // uniform
        int v[4];   // per lane
    };
    auto tile_ids = [&](int ids, TileIds& T) {
#pragma unroll
        for (int p = 0; p < 4; ++p) T.k[p] = __builtin_amdgcn_readlane(ids, kslot[p]);
#pragma unroll
        for (int p = 0; p < 4; ++p) T.v[p] = __builtin_amdgcn_ds_bpermute(vslot[p] << 2, ids);
    };
    // Addresses of tile t's eight loads: K load p reads from ksb[p] + koff[p]
    // (a scalar base), V load p from va[p].
    struct TileAddr {
        const char* ksb[4];
        const char* va[4];
    };
    // Block offsets are ids times the block's bytes, 32 x 32 -> 64 bits (the
    // host checks that the bytes fit 32 bits); V load p's per-lane base is
    // fixed.
    const uint32_t tb32 = static_cast<uint32_t>(tile_bytes);
    const char* vb0[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) vb0[p] = vbase + voff[p];
    auto tile_addr = [&](int t, const TileIds& T, TileAddr& A) {
        // the tile's offset inside its block (only for blocks larger than a tile)
        const int in_blk = big_blocks ? ((t * kKT) & (bs - 1)) : 0;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            A.ksb[p] = kbase + static_cast<uint64_t>(static_cast<uint32_t>(T.k[p])) * tb32 + in_blk * 32 * 2;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            A.va[p] = vb0[p] + static_cast<uint64_t>(static_cast<uint32_t>(T.v[p])) * tb32 + in_blk * 2;
    };
    // LDS destinations of this wave's loads in buffer 0 (buffer 1 is one
    // tile on), computed once: worked out per load, the compiler kept these
    // uniform addresses in vector registers.
    const uint32_t m0k = lds_address(&sK[0][16 * w * kD]);
    const uint32_t m0v = lds_address(&sV[0][32 * w * kKT]);
    // load i of 8 (K loads 0-3, then V loads 0-3) into buffer buf
    auto load_part = [&](const TileAddr& A, int i, int buf) {
        if (i < 4)
            load_to_lds_s(A.ksb[i], koff[i], m0k + (buf * kKT * kD + 4 * i * kD) * 2);
        else
            load_to_lds(A.va[i - 4], m0v + (buf * kD * kKT + 8 * (i - 4) * kKT) * 2);
    };
    f32x16_t acc[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mt][e] = 0.f;
    float m_run = -INFINITY;                      // running max of the row's logits (raw units)
    float l_run = 0.f;                            // this lane's half of the row's weight sum
    const float cscale = a.scale_log2;
    const float lazy = kLazyLog2 / cscale;        // max growth tolerated before a rescale (raw units)
    const int wave_min_pos = P0 + qt * QT + ((32 * w) >> a.log2G);
    const int krow0 = k_row_key(col);             // K row read for A-operand row `col`
    const int kx = krow0 & 15;                    // K swizzle of the rows this lane reads
    const int vx = (col >> 1) & 7;                // V swizzle of the rows this lane reads
    // The direct loads count in vmcnt; a wave's loads have written LDS once it
    // reaches zero (encoding: vmcnt 0, expcnt and lgkmcnt left at their maxima).
    auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };
    // The last tile's values past the context end are zeroed in LDS once it
    // has landed (a weight of 0 does not cancel a NaN); keys there need no
    // care, their logits are masked by the causal test.
    auto zero_v_tail = [&](int buf, int t) {
        const int nval = Lc - t * kKT;            // keys of the tile inside the context
        if (nval >= kKT) return;
        __syncthreads();                          // every wave's share of the tile is in LDS
        // one 16-byte segment (8 keys of one channel row) per item
        for (int item = tid; item < kD * (kKT / 8); item += kThreads) {
            const int d = item / (kKT / 8), s = item % (kKT / 8);
            const int keep = nval - 8 * s;        // keys of the segment inside the context
            if (keep >= 8) continue;
            u32x4* p = reinterpret_cast<u32x4*>(&sV[buf][d * kKT + 8 * (s ^ ((d >> 1) & 7))]);
            *p = keep <= 0 ? kZero4 : keep_first_bf16(*p, keep);
        }
    };

    // ---- prologue: ids of tiles 0 and 1, then tile 0 into LDS ----
    TileIds T;                                    // ids of the next tile to load
    {
        const int r0 = load_raw(0);
        const int r1 = load_raw(min(1, nkt - 1));
        tile_ids(check_ids(0, r0), T);
        TileAddr A;
        tile_addr(0, T, A);
#pragma unroll
        for (int i = 0; i < 8; ++i) load_part(A, i, 0);
        tile_ids(check_ids(min(1, nkt - 1), r1), T);
    }
    wait_loads();
    if (nkt == 1) zero_v_tail(0, 0);
    __syncthreads();

    // Fragment addresses in buffer 0: K fragment of channel step ks (rows of
    // the first 32-key half; the second is 32 rows on), V fragment of key
    // segment group (t, kb) (channel tile 0; tile mt is 32 rows on).  The
    // tile loop is unrolled by two, so the buffer is a constant and every
    // fragment read is one of these addresses plus an immediate offset.
    const uint16_t* kfp[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) kfp[ks] = &sK[0][krow0 * kD + 8 * ((2 * ks + hh) ^ kx)];
    const uint16_t* vfp[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) vfp[t][kb] = &sV[0][col * kKT + 8 * ((hh + 4 * t + 2 * kb) ^ vx)];

    // One key tile kt, read from buffer BUF = kt & 1.
    auto tile = [&](int kt, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        const int base = kt * kKT;
        // Tile kt + 1's eight loads are issued one per channel step of the
        // logits below: issued back to back, the four waves' loads queued
        // behind each other in the memory pipeline and each wave waited
        // there instead of issuing matrix instructions.  In the last
        // iteration they fetch tile nkt - 1 again into the free buffer, so no
        // load sits behind a branch.
        TileAddr A;
        tile_addr(min(kt + 1, nkt - 1), T, A);
        // tile kt + 2's block ids: loaded now, checked after this tile's
        // math, so the wait for them is not on the critical path
        // Every thread loads and checks one id in every iteration (lanes
        // past n_ids, and iterations with no tile kt + 2, repeat an id
        // already read), so the load is always consumed on the same path.
        const int t2 = min(kt + 2, nkt - 1);
        const int raw = load_raw(t2);

        // ---- logits S^T[key][row] for the tile's two 32-key MFMA tiles ----
        // The two 32-key MFMA chains are interleaved (channel step outer), so
        // each K fragment read has two MFMAs of lead time and the two
        // accumulators alternate.
        f32x16_t st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) st[t][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(kfp[ks] + buf * kKT * kD + 32 * t * kD);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), st[t], 0, 0, 0);
            }
            load_part(A, ks, buf ^ 1);
        }
        // Scheduling hint (LDS reads = 0x100, MFMA = 0x008): 4 fragment reads,
        // then (2 MFMAs, 2 reads) x 6, then 4 MFMAs, so each read leads its MFMA
        // by two MFMA pairs instead of one.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // The first 32-key half's V fragments are read now, so that their LDS
        // latency is spent on the mask, the maximum and the weights (read next
        // to their MFMAs, as the compiler placed them, each stalled on its
        // read); the second half's take the same registers once the first
        // half's MFMAs have issued.
        u32x4 vf[kMT][2];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                vf[mt][kb] = *reinterpret_cast<const u32x4*>(vfp[0][kb] + buf * kD * kKT + 32 * mt * kKT);
        __builtin_amdgcn_sched_barrier(0);
        // element e of tile t holds key base + 32 t + 16 (e / 8) + 8 hh + e % 8
        if (base + kKT - 1 > wave_min_pos) {
            // key <= rowpos, with the element's constant part of the key on the left
            const int lim = rowpos - base - 8 * hh;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    st[t][e] = 32 * t + 16 * (e >> 3) + (e & 7) <= lim ? st[t][e] : -INFINITY;
        }
        // ---- online softmax of the row (this lane and lane ^ 32 share it) ----
        float mx = st[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[t][e]);
        mx = fmaxf(mx, other_half(mx));
        const bool grow = mx > m_run + lazy;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * cscale) : 1.f;
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) acc[mt] *= alpha;
        }
        const float neg_m = -m_run * cscale;
        // Weights and values one 32-key half at a time: the value MFMAs of
        // the first half are independent of the second half's exponentials,
        // so the two overlap within the wave.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // weights converted to bf16 in pairs (one conversion per two); the
            // row sum takes the same bf16 weights as the value product, two
            // per instruction
            u32x4 pw[2];
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float2_t x = {__builtin_amdgcn_exp2f(fmaf(st[t][e], cscale, neg_m)),
                                    __builtin_amdgcn_exp2f(fmaf(st[t][e + 1], cscale, neg_m))};
                const bf16x2_t w2 = __builtin_convertvector(x, bf16x2_t);
                pw[e >> 3][(e & 7) >> 1] = __builtin_bit_cast(uint32_t, w2);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(w2, kOnes2, l_run, false);
            }
            const bf16x8_t pb[2] = {as_bf16x8(pw[0]), as_bf16x8(pw[1])};
            // ---- values: O^T[channel][row] += V^T[channel][key] . P^T[key][row] ----
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    // keys base + 8 (hh + 4 t + 2 kb) .. +7 of channel 32 mt + col
                    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[mt][kb]), pb[kb], acc[mt], 0, 0, 0);
                    if (t == 0)
                        vf[mt][kb] = *reinterpret_cast<const u32x4*>(vfp[1][kb] + buf * kD * kKT + 32 * mt * kKT);
                }
            }
        }
        // the wait for tile kt + 1's loads stays behind every value MFMA
        __builtin_amdgcn_sched_barrier(0);
        wait_loads();                             // this wave's share of tile kt + 1 is in LDS
        // The id of tile kt + 2 was loaded after tile kt + 1's loads, so its
        // check needs them all to have landed: keep it behind the wait, where
        // the scheduler cannot hoist it (and the wait with it) into the value
        // products above.
        __builtin_amdgcn_sched_barrier(0);
        tile_ids(check_ids(t2, raw), T);
        if (kt + 2 == nkt) zero_v_tail(buf ^ 1, kt + 1);
        __syncthreads();
    };
    for (int kt = 0; kt < nkt; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < nkt) tile(kt + 1, std::integral_constant<int, 1>{});
    }
    // bad is the same in every wave: each checks the same ids

    // ---- normalise and store: lane holds channels 32 mt + 8 (e / 4) + 4 hh + e % 4 of its row ----
    const float l_tot = l_run + other_half(l_run);
    if (!rowok) return;
    const int64_t orow = (static_cast<int64_t>(qs0 + qi) * a.Hq + g * G + (rho & (G - 1))) * kD;
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            f32x4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = bad ? kNaN : acc[mt][4 * e4 + i] * inv;
            const int64_t o = orow + 32 * mt + 8 * e4 + 4 * hh;
            if (a.out_bf16) {
                __bf16* dst = static_cast<__bf16*>(a.out) + o;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = static_cast<__bf16>(v[i]);
            } else {
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + o) = v;
            }
        }
}

}  // namespace
}  // namespace pa

extern "C" int pa_prefill(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                          const void* v_cache, const pa_cache_desc* desc, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_chunks, int32_t num_query_tokens,
                          int32_t num_q_heads, int32_t max_query_len, float scale, void* stream) {
    using namespace pa;
    if (!desc_ok(desc) || num_chunks < 0 || num_query_tokens < 0 || num_q_heads <= 0 ||
        max_query_len < 0 || max_blocks_per_seq < 0)
        return PA_ERR_INVALID_ARG;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    // The running max is kept on unscaled logits and raised lazily by
    // 8 / (scale log2 e): that needs a positive, finite scale.
    if (!(scale > 0.f) || !std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    const int32_t H = desc->num_kv_heads;
    if (num_q_heads % H) return PA_ERR_INVALID_ARG;
    const int32_t G = num_q_heads / H;
    if (desc->kv_dtype != PA_BF16 || desc->head_dim != kD) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(G) || G > 16) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(desc->block_size) || desc->block_size < kMinBlock || desc->block_size > 256)
        return PA_ERR_UNSUPPORTED;
    // one block of all kv heads (the stride between blocks) must fit 32 bits
    if (static_cast<int64_t>(H) * desc->block_size * kD * 2 > static_cast<int64_t>(UINT32_MAX))
        return PA_ERR_UNSUPPORTED;
    if (num_chunks == 0 || max_query_len == 0 || num_query_tokens == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
        return PA_ERR_INVALID_ARG;
    // 16-byte loads of q and of the pools
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache)) % 16)
        return PA_ERR_INVALID_ARG;
    int log2G = 0;
    while ((1 << log2G) < G) ++log2G;
    const int QT = kRows / G;
    const int64_t nqt = (max_query_len + QT - 1) / QT;
    // every XCD gets the same number of workgroups: ceil(pairs / 8) pairs'
    // worth; the surplus ones of the XCDs with a pair fewer exit at once
    const int64_t pairs = static_cast<int64_t>(num_chunks) * H;
    const int64_t units = kNumXcds * ((pairs + kNumXcds - 1) / kNumXcds) * nqt;
    if (units > INT32_MAX) return PA_ERR_UNSUPPORTED;
    PrefillArgs a;
    a.out = out;
    a.q = static_cast<const uint16_t*>(q);
    a.kc = static_cast<const uint16_t*>(k_cache);
    a.vc = static_cast<const uint16_t*>(v_cache);
    a.tables = block_tables;
    a.lens = context_lens;
    a.qsl = query_start_loc;
    a.num_chunks = num_chunks;
    a.Hq = num_q_heads;
    a.H = H;
    a.G = G;
    a.log2G = log2G;
    a.bs = desc->block_size;
    int log2bs = 0;
    while ((1 << log2bs) < a.bs) ++log2bs;
    a.log2bs = log2bs;
    a.N = desc->num_blocks;
    a.maxb = max_blocks_per_seq;
    a.max_q = max_query_len;
    a.nqt = static_cast<int32_t>(nqt);
    a.total_q = num_query_tokens;
    a.scale_log2 = scale * kLog2e;
    a.out_bf16 = out_dtype == PA_BF16;
    return launch_kernel(prefill_kernel, dim3(static_cast<uint32_t>(units)), dim3(kThreads), 0,
                         static_cast<hipStream_t>(stream), a);
}
