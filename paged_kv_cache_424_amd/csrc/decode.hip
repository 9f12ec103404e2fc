// Paged decode attention for gfx950: split-K partitions + a rescaling reduce.
//
// What is computed: for every sequence s and query head h, attention of the
// one new query over the sequence's whole context, read block by block through
// its block table ([studynote 223] "KV Cache PagedAttention", three-line summary
// item 3 and section II figure; [ch.09] "09. PagedAttention", section 해법: the
// request sees contiguous logical blocks, the blocks themselves are scattered).
// Paging changes where K/V live, not the result, so the kernels must reach
// softmax(scale * K q) V of the gathered context.
//
// Work decomposition.  One workgroup (4 waves) per (sequence, kv head,
// partition of PART = 128 * NCH tokens).  Wave w takes the 32-token chunks
// w, w+4, w+8, ... of the partition, so a short last partition still spreads
// over the waves.  Each wave keeps an online softmax (running max m, sum l and
// unnormalised output) per query head of the kv head's group; the four waves
// are merged through LDS at the end.  A sequence with one partition gets its
// output here; longer ones leave (m, l, output) per partition in the
// workspace for the reduce kernel.
//
// Matrix cores.  The query group (G <= 16 heads) against a 16-token K tile is
// a dense contraction, done as S^T[token][head] = K[token][:] . Q^T with
// v_mfma_f32_16x16x32_bf16 (fp32: v_mfma_f32_16x16x4_f32).  The value pass is
// done transposed too, O^T[channel][head] = V^T[channel][token] . P^T, so that
// (a) a lane's softmax weights are exactly the B operand it needs -- lane
// (j, r) holds head r's weights of tokens 8j..8j+7 of the chunk -- and (b) the
// per-head rescale of the running output is lane-local (columns are heads).
// The K tile rows are permuted (row r of tile t is token 8(r/4) + r%4 + 4t) to
// line the QK output up with that operand.  V is stored channel-major inside a
// block so that the 8 consecutive tokens of one channel are one 16-byte load.
// bf16 weights are fed to the value MFMA as a hi + lo pair of bf16 numbers, so
// the product keeps ~16 bits of the fp32 weight (one extra MFMA per step; the
// kernel is bound by HBM, not by the matrix cores).
//
// Every (s, h) result depends only on logical positions, never on physical
// block ids, and uses no atomics: outputs are bit-identical under any
// relabelling of blocks and whether a prefix is shared or duplicated.

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;       // tokens per wave step

struct DecodeArgs {
    void* out;
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* tables;
    const int32_t* lens;
    float* ws_acc;     // [B][Hq][P][D]
    float2* ws_ml;     // [B][Hq][P] (max in log2 units, sum)
    int32_t B, Hq, H, G, bs, N, maxb, max_ctx, P;
    float scale_log2;  // scale * log2(e): logits are kept in base-2 units
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

template <bool BF16, int D, int NCH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void decode_partition_kernel(
    DecodeArgs a) {
    constexpr int PART = kChunk * kWaves * NCH;
    constexpr int ES = BF16 ? 2 : 4;
    using Regs = ChunkRegs<BF16, D>;
    constexpr int MT = D / 16;                    // output channel tiles

    const int u = xcd_remap(blockIdx.x, gridDim.x);
    const int s = u % a.B;
    const int pg = u / a.B;
    const int p = pg % a.P;
    const int g = pg / a.P;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int r = lane & 15;
    const int j = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.G;

    const int L = a.lens[s];
    const bool bad_len = L < 1 || L > a.max_ctx || static_cast<int64_t>(L) > static_cast<int64_t>(a.maxb) * a.bs;
    const int nparts = bad_len ? 1 : (L + PART - 1) / PART;
    if (p >= nparts) return;

    const float kNaN = __builtin_nanf("");
    if (bad_len) {
        // Invalid length: NaN for the group's heads, nothing read.
        for (int e = tid; e < G * D; e += kThreads) {
            const int h = e / D, d = e % D;
            store_out(a.out, (static_cast<int64_t>(s) * a.Hq + g * G + h) * D + d, kNaN, a.out_bf16);
        }
        return;
    }

    // Block ids of this partition, validated once: a bad id makes the whole
    // group's output NaN and is never dereferenced.
    __shared__ int s_blk[PART / 4];
    const int bs = a.bs;
    const int nbp = PART / bs;                    // blocks per partition (bs divides PART)
    const int nblk_seq = (L + bs - 1) / bs;
    int bad = 0;
    for (int i = tid; i < nbp; i += kThreads) {
        const int b = p * nbp + i;
        int id = 0;
        if (b < nblk_seq) {
            id = a.tables[static_cast<int64_t>(s) * a.maxb + b];
            if (id < 0 || id >= a.N) {
                bad = 1;
                id = 0;
            }
        }
        s_blk[i] = id;
    }
    bad = __syncthreads_or(bad);

    const int64_t tile_elems = static_cast<int64_t>(a.H) * bs * D;   // one block, all heads
    const char* kbase = static_cast<const char*>(a.kc) + static_cast<int64_t>(g) * bs * D * ES;
    const char* vbase = static_cast<const char*>(a.vc) + static_cast<int64_t>(g) * D * bs * ES;

    // Query operand: lane (j, r) holds head r's channels for k-group j.
    constexpr int QV = BF16 ? D / 32 : D / 16;
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

    const int part0 = p * PART;                   // first absolute position of the partition

    // Loads are unconditional: every address is inside the pool (ids of blocks
    // past the sequence's end were replaced by block 0 above), so no load sits
    // behind a divergent branch and all of a chunk's loads issue back to back.
    // Rows past the context end are dealt with when the chunk is consumed: their
    // logits are selected to -inf and their values to 0.
    auto load_chunk = [&](int ci, Regs& R) {
        const int tc = ci * kChunk;               // chunk offset inside the partition
        // K: row r of tile t is chunk token 8*(r>>2) + (r&3) + 4t.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int tp = tc + 8 * (r >> 2) + (r & 3) + 4 * t;
            const int64_t blk = s_blk[tp / bs];
            const char* row = kbase + ((blk * tile_elems) + static_cast<int64_t>(tp % bs) * D) * ES;
#pragma unroll
            for (int c = 0; c < Regs::KV; ++c) {
                const int d0 = BF16 ? c * 32 + j * 8 : j * (D / 4) + 4 * c;
                R.k[t][c] = ldg_nt(row + static_cast<int64_t>(d0) * ES);
            }
        }
        // V: lane (j, r) reads tokens 8j..8j+7 of channel mt*16 + r.
        const int tp0 = tc + 8 * j;
        const int64_t blk = s_blk[tp0 / bs];
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

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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
                        c4 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kk[e]), __uint_as_float(qq[e]),
                                                                  c4, 0, 0, 0);
                }
            }
            st[t] = c4;
        }
        // lane (j, r): head r, chunk tokens 8j + e with e = 4t + i
        float sv[8];
        const int ntok = L - (part0 + tc + 8 * j);         // valid tokens among this lane's 8
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
        // the chunk holds at least one valid token, so cm is finite
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
        if (part0 + tc + kChunk > L) {
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
                const __bf16 h = static_cast<__bf16>(pv[e]);
                ph[e] = h;
                pl[e] = static_cast<__bf16>(pv[e] - static_cast<float>(h));
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
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(e < 4 ? v0[e] : v1[e - 4]), pv[e],
                                                                   acc[mt], 0, 0, 0);
            }
        }
    };

    // Chunk loop.  Latency is hidden by occupancy, not by an explicit register
    // double buffer: the kernel is held to >= 3 waves per SIMD (at most ~168
    // registers each), which leaves the scheduler room to start a chunk's
    // sixteen 16-byte loads early while keeping three workgroups resident per
    // CU -- one workgroup's start-up (length, block ids, query) and merge then
    // overlap the others' streaming.  An explicit two-chunk buffer needs ~260
    // registers and one wave per SIMD, and measured 25 % slower.
    const int first_empty = (L - part0 + kChunk - 1) / kChunk;   // chunks >= this are empty
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int ci = w + kWaves * k;
        if (ci >= first_empty) break;
        Regs R;
        load_chunk(ci, R);
        compute_chunk(ci, R);
    }

    // ---- merge the four waves through LDS ----
    extern __shared__ float s_dyn[];
    const int rowstride = D + 4;
    float* s_acc = s_dyn;                                   // [4][G][D+4]
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (j == 0) {
        s_m[w][r] = m_run;
        s_l[w][r] = l_tot;
    }
    if (r < G) {
        float* dst = s_acc + (w * G + r) * rowstride;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[mt * 16 + 4 * j + i] = acc[mt][i];
    }
    __syncthreads();

    const bool single = nparts == 1;
    for (int e = tid; e < G * D; e += kThreads) {
        const int h = e / D, d = e % D;
        float M = s_m[0][h];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = __builtin_amdgcn_exp2f(s_m[ww][h] - M);
            o += f * s_acc[(ww * G + h) * rowstride + d];
            l += f * s_l[ww][h];
        }
        const int64_t sh = static_cast<int64_t>(s) * a.Hq + g * G + h;
        if (single) {
            store_out(a.out, sh * D + d, bad ? kNaN : o / l, a.out_bf16);
        } else {
            a.ws_acc[(sh * a.P + p) * D + d] = bad ? kNaN : o;
            if (d == 0) a.ws_ml[sh * a.P + p] = bad ? make_float2(kNaN, kNaN) : make_float2(M, l);
        }
    }
}

// One workgroup per (sequence, query head): merge the partitions of a
// sequence that has more than one.  With M the largest partition max, each
// partition's sum and output are weighted by 2^(m_p - M); the result is their
// ratio.  Thread t owns channel t % D and the partitions p = t / D (mod 256/D);
// the partial sums are combined through LDS in a fixed order, so the result
// does not depend on timing.
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

__global__ __launch_bounds__(256) void decode_reduce_kernel(void* out, int out_bf16,
                                                           const int32_t* __restrict__ lens,
                                                           const float* __restrict__ ws_acc,
                                                           const float2* __restrict__ ws_ml, int32_t B,
                                                           int32_t Hq, int32_t D, int32_t max_ctx,
                                                           int32_t part, int32_t P) {
    const int pair = blockIdx.x;
    const int s = pair / Hq;
    const int L = lens[s];
    if (L < 1 || L > max_ctx) return;                       // the partition kernel wrote NaN
    const int np = (L + part - 1) / part;
    if (np <= 1) return;                                    // already final
    __shared__ float red[4];
    __shared__ float s_part[256];
    const int tid = threadIdx.x;
    const float2* ml = ws_ml + static_cast<int64_t>(pair) * P;
    float m = -INFINITY;
    for (int i = tid; i < np; i += 256) m = fmaxf(m, ml[i].x);
    const float M = block_reduce(m, red, true);
    float dp = 0.f;
    for (int i = tid; i < np; i += 256) {
        const float2 v = ml[i];
        dp += __builtin_amdgcn_exp2f(v.x - M) * v.y;
    }
    const float den = block_reduce(dp, red, false);

    const int groups = 256 / D;                             // D divides 256
    const int d = tid % D, grp = tid / D;
    const float* accp = ws_acc + static_cast<int64_t>(pair) * P * D + d;
    // four independent partial sums keep four loads in flight per thread
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    int i = grp;
    for (; i + 3 * groups < np; i += 4 * groups) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pi = i + u * groups;
            o[u] += __builtin_amdgcn_exp2f(ml[pi].x - M) * accp[static_cast<int64_t>(pi) * D];
        }
    }
    for (int u = 0; i < np; i += groups, ++u)
        o[u] += __builtin_amdgcn_exp2f(ml[i].x - M) * accp[static_cast<int64_t>(i) * D];
    const float o0 = o[0] + o[2], o1 = o[1] + o[3];
    s_part[tid] = o0 + o1;
    __syncthreads();
    if (grp == 0) {
        float o = s_part[d];
        for (int g2 = 1; g2 < groups; ++g2) o += s_part[g2 * D + d];
        const float v = o / den;
        const int64_t idx = static_cast<int64_t>(pair) * D + d;
        if (out_bf16)
            static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);
        else
            static_cast<float*>(out)[idx] = v;
    }
}

struct Checked {
    int32_t part;
    int32_t P;
    int32_t G;
};

int check_decode(const pa_cache_desc* desc, int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads,
                 int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                 Checked* c) {
    if (!desc_ok(desc) || num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 ||
        max_context_len < 1)
        return PA_ERR_INVALID_ARG;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    const int32_t H = desc->num_kv_heads;
    if (num_q_heads % H) return PA_ERR_INVALID_ARG;
    const int32_t G = num_q_heads / H;
    const int32_t part = partition_size == 0 ? 512 : partition_size;
    if (part < 128 || part > 512 || part % 128) return PA_ERR_UNSUPPORTED;
    const int32_t bs = desc->block_size;
    if (!is_pow2(bs) || bs < 8 || bs > part) return PA_ERR_UNSUPPORTED;
    if (G > 16) return PA_ERR_UNSUPPORTED;
    if (desc->head_dim != 64 && desc->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * bs)
        return PA_ERR_INVALID_ARG;
    c->part = part;
    c->P = (max_context_len + part - 1) / part;
    c->G = G;
    return PA_OK;
}

size_t workspace_bytes(int64_t B, int64_t Hq, int64_t D, int64_t P) {
    if (P <= 1) return 0;
    const int64_t acc = B * Hq * P * D * 4;
    const int64_t acc_aligned = (acc + 255) / 256 * 256;
    return static_cast<size_t>(acc_aligned + B * Hq * P * 8);
}

template <bool BF16, int D>
int launch_partitions_nch(int nch, dim3 grid, size_t lds, hipStream_t st, const DecodeArgs& a) {
    switch (nch) {
        case 1: return launch_kernel(decode_partition_kernel<BF16, D, 1>, grid, dim3(kThreads), lds, st, a);
        case 2: return launch_kernel(decode_partition_kernel<BF16, D, 2>, grid, dim3(kThreads), lds, st, a);
        case 3: return launch_kernel(decode_partition_kernel<BF16, D, 3>, grid, dim3(kThreads), lds, st, a);
        case 4: return launch_kernel(decode_partition_kernel<BF16, D, 4>, grid, dim3(kThreads), lds, st, a);
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
    const int32_t part = partition_size == 0 ? 512 : partition_size;
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 1 || part <= 0) return 0;
    const int64_t P = (static_cast<int64_t>(max_context_len) + part - 1) / part;
    return pa::workspace_bytes(num_seqs, num_q_heads, head_dim, P);
}

int pa_decode_partitions(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                         const void* v_cache, const pa_cache_desc* desc,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_context_len, float scale, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, void* stream) {
    using namespace pa;
    Checked c;
    int rc = check_decode(desc, out_dtype, num_seqs, num_q_heads, max_blocks_per_seq, max_context_len,
                          partition_size, &c);
    if (rc != PA_OK) return rc;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
    const int32_t D = desc->head_dim;
    const size_t need = pa::workspace_bytes(num_seqs, num_q_heads, D, c.P);
    if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_INVALID_ARG;
    const int64_t units = static_cast<int64_t>(num_seqs) * desc->num_kv_heads * c.P;
    if (units > INT32_MAX) return PA_ERR_UNSUPPORTED;

    DecodeArgs a;
    a.out = out;
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = context_lens;
    const int64_t acc_bytes = static_cast<int64_t>(num_seqs) * num_q_heads * c.P * D * 4;
    a.ws_acc = static_cast<float*>(workspace);
    a.ws_ml = need ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + (acc_bytes + 255) / 256 * 256)
                   : nullptr;
    a.B = num_seqs;
    a.Hq = num_q_heads;
    a.H = desc->num_kv_heads;
    a.G = c.G;
    a.bs = desc->block_size;
    a.N = desc->num_blocks;
    a.maxb = max_blocks_per_seq;
    a.max_ctx = max_context_len;
    a.P = c.P;
    a.scale_log2 = scale * kLog2e;
    a.out_bf16 = out_dtype == PA_BF16;

    const dim3 grid(static_cast<uint32_t>(units));
    const size_t lds = static_cast<size_t>(kWaves) * c.G * (D + 4) * sizeof(float);
    const int nch = c.part / (kChunk * kWaves);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (desc->kv_dtype == PA_BF16)
        return D == 128 ? launch_partitions_nch<true, 128>(nch, grid, lds, st, a)
                        : launch_partitions_nch<true, 64>(nch, grid, lds, st, a);
    return D == 128 ? launch_partitions_nch<false, 128>(nch, grid, lds, st, a)
                    : launch_partitions_nch<false, 64>(nch, grid, lds, st, a);
}

int pa_decode_reduce(void* out, int32_t out_dtype, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace pa;
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 1) return PA_ERR_INVALID_ARG;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    const int32_t part = partition_size == 0 ? 512 : partition_size;
    if (part < 128 || part > 512 || part % 128) return PA_ERR_UNSUPPORTED;
    const int32_t P = (max_context_len + part - 1) / part;
    const size_t need = pa::workspace_bytes(num_seqs, num_q_heads, head_dim, P);
    if (need == 0 || num_seqs == 0) return PA_OK;        // every sequence fits one partition
    if (!out || !context_lens || !workspace || workspace_bytes < need) return PA_ERR_INVALID_ARG;
    const int64_t pairs = static_cast<int64_t>(num_seqs) * num_q_heads;
    const int64_t acc_bytes = pairs * P * head_dim * 4;
    const float* ws_acc = static_cast<const float*>(workspace);
    const float2* ws_ml =
        reinterpret_cast<const float2*>(static_cast<const char*>(workspace) + (acc_bytes + 255) / 256 * 256);
    const int64_t grid = pairs;
    if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
    return launch_kernel(decode_reduce_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                         static_cast<hipStream_t>(stream), out, out_dtype == PA_BF16, context_lens,
                         ws_acc, ws_ml, num_seqs, num_q_heads, head_dim, max_context_len, part, P);
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
