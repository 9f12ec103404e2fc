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
// 256 rows), a row being one (query position, query head of the kv head's
// group): 256/G positions x G heads.  The workgroup walks the key positions in
// tiles of 32; each tile's K rows and V channel rows are copied from their
// physical blocks into LDS (double buffered, one barrier per tile) and shared
// by the four waves.  Each wave owns 64 rows (four 16-row MFMA column tiles),
// holds their query fragments in registers for the whole walk, and keeps an
// online softmax per row.
//
// Matrix cores, as in the decode kernel: S^T[key][row] = K . Q^T and
// O^T[channel][row] += V^T . P^T with v_mfma_f32_16x16x32_bf16, so a lane's
// softmax weights (row n, keys 8j..8j+7 of the tile) are exactly its operand
// for the value MFMA and the per-row rescale is lane-local.  Weights enter
// the value MFMA as bf16 (8-bit mantissa; the accumulation is fp32).  Per
// 32-key tile a wave issues 64 MFMAs (16 cycles each) against 16 KB of LDS
// reads, so the matrix cores, not LDS or HBM, set the pace.  LDS rows are
// padded by 16 bytes so the 16 lanes of a quarter-wave read 16 different
// bank groups.

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 32;                 // keys per tile
constexpr int kNT = 4;                    // 16-row column tiles per wave
constexpr int kRows = 16 * kNT * kWaves;  // 256 rows per workgroup
constexpr int kD = 128;
constexpr int kMT = kD / 16;              // channel tiles of the output
constexpr int kKS = kD / 32;              // k-steps of the logits MFMA
constexpr int kKStride = kD + 8;          // bf16 per K row in LDS (272 bytes)
constexpr int kVStride = kKeys + 8;       // bf16 per V channel row in LDS (80 bytes)

struct PrefillArgs {
    void* out;
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* tables;
    const int32_t* lens;
    const int32_t* qsl;
    int32_t num_chunks, Hq, H, G, log2G, bs, N, maxb, max_q, nqt, total_q;
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

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(
    PrefillArgs a) {
    __shared__ __align__(16) uint16_t sK[2][kKeys * kKStride];
    __shared__ __align__(16) uint16_t sV[2][kD * kVStride];

    const int u = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = a.nqt - 1 - (u % a.nqt);       // longest query tiles of a chunk first
    const int cg = u / a.nqt;
    const int g = cg % a.H;
    const int c = cg / a.H;
    const int G = a.G;
    const int QT = kRows >> a.log2G;              // query positions per tile

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = lane & 15;
    const int j = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int qs0 = a.qsl[c];
    const int Cc = a.qsl[c + 1] - qs0;
    const int Lc = a.lens[c];
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
    const int nkt = (P0 + qhi + kKeys - 1) / kKeys;            // key tiles to visit

    // ---- query fragments: lane (j, n) of column tile nt holds row 64w + 16nt + n ----
    u32x4 qf[kNT][kKS];
    int rowpos[kNT];                                           // absolute position of the row
    bool rowok[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int rho = 64 * w + 16 * nt + n;
        const int qi = qt * QT + (rho >> a.log2G);
        const int h = rho & (G - 1);
        rowok[nt] = qi < Cc;
        rowpos[nt] = P0 + qi;
        const uint16_t* qrow = a.q + (static_cast<int64_t>(qs0 + (rowok[nt] ? qi : 0)) * a.Hq + g * G + h) * kD;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + ks * 32 + j * 8);
            qf[nt][ks] = rowok[nt] ? x : kZero4;
        }
    }

    // ---- tile loader: each thread moves 2 K segments and 2 V segments of 16 bytes ----
    const int64_t tile_elems = static_cast<int64_t>(a.H) * a.bs * kD;
    const int32_t* trow = a.tables + static_cast<int64_t>(c) * a.maxb;
    const int nblk = (Lc + a.bs - 1) / a.bs;
    int bad = 0;
    auto block_of = [&](int key) -> int64_t {
        const int b = key / a.bs;
        if (b >= nblk) return 0;                 // past the context: any valid block, masked later
        const int id = trow[b];
        if (id < 0 || id >= a.N) {
            bad = 1;
            return 0;
        }
        return id;
    };
    u32x4 pk[2], pv[2];
    auto load_tile = [&](int kt) {
        const int base = kt * kKeys;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int key = (tid >> 4) + 16 * p, seg = tid & 15;
            const int kk = base + key;
            const int64_t blk = block_of(kk);
            pk[p] = *reinterpret_cast<const u32x4*>(
                a.kc + ((blk * tile_elems) + (static_cast<int64_t>(g) * a.bs + kk % a.bs) * kD) + seg * 8);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int d = (tid >> 2) + 64 * p, sg = tid & 3;
            const int kk0 = base + 8 * sg;
            const int64_t blk = block_of(kk0);
            const u32x4 x = *reinterpret_cast<const u32x4*>(
                a.vc + (blk * tile_elems + (static_cast<int64_t>(g) * kD + d) * a.bs + kk0 % a.bs));
            const int nval = Lc - kk0;                       // values past the context are zeroed
            pv[p] = nval >= 8 ? x : keep_first_bf16(x, nval);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int key = (tid >> 4) + 16 * p, seg = tid & 15;
            *reinterpret_cast<u32x4*>(&sK[buf][key * kKStride + seg * 8]) = pk[p];
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int d = (tid >> 2) + 64 * p, sg = tid & 3;
            *reinterpret_cast<u32x4*>(&sV[buf][d * kVStride + 8 * sg]) = pv[p];
        }
    };

    f32x4_t acc[kNT][kMT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[kNT], l_run[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
    }
    const int wave_min_pos = P0 + qt * QT + ((64 * w) >> a.log2G);   // smallest position of this wave's rows

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const int base = kt * kKeys;
        if (kt + 1 < nkt) load_tile(kt + 1);

        // ---- logits S^T[key][row]; key row r of tile t is key 8(r/4) + r%4 + 4t ----
        f32x4_t st[2][kNT];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int krow = 8 * (n >> 2) + (n & 3) + 4 * t;
            u32x4 kf[kKS];
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks)
                kf[ks] = *reinterpret_cast<const u32x4*>(&sK[buf][krow * kKStride + ks * 32 + j * 8]);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < kKS; ++ks)
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[ks]), as_bf16x8(qf[nt][ks]), s4, 0, 0, 0);
                st[t][nt] = s4;
            }
        }
        // ---- online softmax per row; lane (j, n) holds keys base + 8j + e ----
        const bool diag = base + kKeys - 1 > wave_min_pos;   // some key may lie after some row
        bf16x8_t pb[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            float sv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = st[e >> 2][nt][e & 3] * a.scale_log2;
                sv[e] = (!diag || base + 8 * j + e <= rowpos[nt]) ? x : -INFINITY;
            }
            float cm = sv[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) cm = fmaxf(cm, sv[e]);
            cm = fmaxf(cm, __shfl_xor(cm, 16));
            cm = fmaxf(cm, __shfl_xor(cm, 32));
            const float m_new = fmaxf(m_run[nt], cm);         // finite: key 0 <= every position
            const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
            m_run[nt] = m_new;
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(sv[e] - m_new);
                ps += pe;
                pb[nt][e] = static_cast<__bf16>(pe);
            }
            l_run[nt] = l_run[nt] * alpha + ps;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) acc[nt][mt] *= alpha;
            }
        }
        // ---- values: O^T[channel][row] += V^T[channel][key] . P^T[key][row] ----
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const u32x4 vf = *reinterpret_cast<const u32x4*>(&sV[buf][(mt * 16 + n) * kVStride + 8 * j]);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), pb[nt], acc[nt][mt], 0, 0, 0);
        }
        if (kt + 1 < nkt) store_tile(buf ^ 1);
        __syncthreads();
    }
    bad = __syncthreads_or(bad);

    // ---- normalise and store: lane (j, n) holds channels mt*16 + 4j .. +3 of its row ----
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        float l = l_run[nt] + __shfl_xor(l_run[nt], 16);
        l += __shfl_xor(l, 32);
        if (!rowok[nt]) continue;
        const int rho = 64 * w + 16 * nt + n;
        const int qi = qt * QT + (rho >> a.log2G);
        const int64_t orow = (static_cast<int64_t>(qs0 + qi) * a.Hq + g * G + (rho & (G - 1))) * kD;
        const float inv = 1.f / l;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            f32x4_t v = acc[nt][mt] * inv;
            if (bad) v = f32x4_t{kNaN, kNaN, kNaN, kNaN};
            const int64_t o = orow + mt * 16 + 4 * j;
            if (a.out_bf16) {
                __bf16* dst = static_cast<__bf16*>(a.out) + o;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = static_cast<__bf16>(v[i]);
            } else {
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + o) = v;
            }
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
    const int32_t H = desc->num_kv_heads;
    if (num_q_heads % H) return PA_ERR_INVALID_ARG;
    const int32_t G = num_q_heads / H;
    if (desc->kv_dtype != PA_BF16 || desc->head_dim != kD) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(G) || G > 16) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(desc->block_size) || desc->block_size < 8 || desc->block_size > 256) return PA_ERR_UNSUPPORTED;
    if (num_chunks == 0 || max_query_len == 0 || num_query_tokens == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
        return PA_ERR_INVALID_ARG;
    int log2G = 0;
    while ((1 << log2G) < G) ++log2G;
    const int QT = kRows / G;
    const int64_t nqt = (max_query_len + QT - 1) / QT;
    const int64_t units = static_cast<int64_t>(num_chunks) * H * nqt;
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
