// Short-query attention over a quantized KV cache (decode) for CDNA4 (gfx950).
//
// The cache holds the K/V half of the prep step (smoothed INT8 K with its
// scales; V as E4M3 code bytes, or binary16 for the binary16 P.V), quantized
// once.  E4M3 V tiles stay one byte per value in LDS and are converted to
// binary16 (exactly) as each P.V fragment is read, so a block moves 2 bytes
// per K+V element pair from HBM and LDS holds a work-group for each of the
// CU's four SIMDs (three with binary16 V).  A short
// query -- Nq rows per q head, sitting at the last Nq of the Nk positions --
// attends to it with the same per-block computation as the prefill kernel
// (attn_block.h).  The query rows are quantized here, one INT8 scale per row.
//
// Work decomposition (flash-decoding): one work-group is one wave, and owns 32
// packed query rows of one (batch, kv head) -- the G q heads that share the kv
// head times the Nq rows, so K and V are read once for all of them -- and one
// chunk of consecutive key blocks.  Each chunk leaves its (reference max, row
// sum, unnormalised O) per row; decode_merge combines the chunks of a row with
// weights 2^(reference max - overall max), a third accumulation level in FP32
// over the two of the block computation.  With a single chunk the kernel
// writes the output itself.
#include "attn_block.h"

namespace sage {

struct DecodeArgs {
    const uint16_t* q;      // [B, Hq, Nq, d], fp16 or bf16 bits
    const int8_t* k_i8;     // cache, [B, Hkv, Np, d]
    const float* k_scale;   // [B, Hkv, Np / k_block]
    const void* v;          // [B, Hkv, Np / SAGE_BN, d, SAGE_BN], E4M3 bytes or binary16
    const float* v_scale;   // [B, Hkv, d]
    float* out;             // [B, Hq, Nq, d]
    float* part_o;          // [B * Hq * Nq, nchunk, d]
    float* part_ml;         // [B * Hq * Nq, nchunk, 2]: reference max, row sum
    int B, Hq, Hkv, Nq, Nk, Np, G;
    int rows_per_head;      // G * Nq packed rows per kv head
    int row_tiles;          // ceil(rows_per_head / 32)
    int nchunk, chunk_blocks;
    float qk, l448;
};

// This lane's part of one query row: elements [32 ks + 16 h, +16) for each
// ks, i.e. exactly the bytes of its Q.K^T operand (zeros for a padding lane).
template <int D>
__device__ inline void load_q_row(const uint16_t* __restrict__ qrow, bool valid, int h,
                                  uint4 (&raw)[D / 16]) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        const int ks = j >> 1, half = j & 1;
        raw[j] = valid ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 16 * h + 8 * half)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
}

// INT8 codes of the row, with one scale for the row; the two lanes of a row
// agree on its absmax through one permlane32 swap.  The codes and the scale
// use the float32 operations of the prep step: scale = absmax / 127, codes
// rne(x * (127 / absmax)) clamped to +-127.
template <typename In, int D>
__device__ inline float quantize_q_row(const uint4 (&raw)[D / 16], v4i (&qf)[D / 32]) {
    constexpr int KS = D / 32;
    float x[KS][16];
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        float f[8];
        unpack8<In>(raw[j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[j >> 1][8 * (j & 1) + e] = f[e];
            am = fmaxf(am, fabsf(f[e]));
        }
    }
    // non-negative floats order like their bit patterns
    am = __builtin_bit_cast(float, max_across_halves(__builtin_bit_cast(int, am)));
    const float inv = am > 0.0f ? 127.0f / am : 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        int w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float r = __builtin_rintf(x[ks][e] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            w[e >> 2] |= ((int)(uint8_t)(int8_t)(int)r) << (8 * (e & 3));
        }
        const v4i c = {w[0], w[1], w[2], w[3]};
        qf[ks] = c;
    }
    return am / 127.0f;
}

// V element bytes in the cache: binary16 for the binary16 P.V, else E4M3.
template <bool PV16>
constexpr int cache_vb() {
    return PV16 ? 2 : 1;
}

// LDS tile buffers per work-group.  A decode wave needs more than half the
// register file, so a CU runs at most one per SIMD, four in all; at d = 128 a
// second buffer would leave LDS for only two of them.  With one buffer per
// tile, the next block's K tile is copied once this block's K fragments are
// read and its V tile once this block's products have read theirs.  (A second
// V buffer at d = 128, with three work-groups per CU, measured slower.)
template <int D>
constexpr int decode_kbufs() {
    return D == 128 ? 1 : 2;
}
template <int D, bool PV16>
constexpr int decode_vbufs() {
    return D == 128 ? 1 : 2;
}
constexpr int kDecodeWavesPerCU = 4;

template <int D, bool PV16>
constexpr size_t decode_lds() {
    return (size_t)decode_kbufs<D>() * SAGE_BN * D +
           (size_t)decode_vbufs<D, PV16>() * D * SAGE_BN * cache_vb<PV16>();
}

// Work-groups resident per CU: four (one per SIMD) where LDS allows; three
// with binary16 V tiles (48 KB).  The key split sizes its grid to this.
template <int D, bool PV16>
constexpr int decode_wgs_per_cu() {
    return 160 * 1024 / decode_lds<D, PV16>() < 4 ? (int)(160 * 1024 / decode_lds<D, PV16>()) : 4;
}

template <typename In, int D, int KSPLIT, bool CAUSAL, bool PV16>
__global__ __launch_bounds__(64) void attn_decode(DecodeArgs a) {
    constexpr int CT = D / 32;
    constexpr int VB = cache_vb<PV16>();
    constexpr bool V8 = VB == 1;
    constexpr int NBUF = decode_kbufs<D>();
    constexpr int NVB = decode_vbufs<D, PV16>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* const lk0 = smem;
    uint8_t* const lk1 = smem + (NBUF - 1) * SAGE_BN * D;
    uint8_t* const lv0 = smem + NBUF * SAGE_BN * D;
    uint8_t* const lv1 = lv0 + (NVB - 1) * D * SAGE_BN * VB;

    const int lane = threadIdx.x;
    const int h = lane >> 5, r32 = lane & 31;
    const v8h rsel = row_sum_selector(lane);

    // work-group -> (batch and kv head, chunk, row tile); row tiles of one
    // chunk are neighbours so they meet the same K/V tiles in the cache
    int idx = blockIdx.x;
    const int rt = idx % a.row_tiles;
    idx /= a.row_tiles;
    const int chunk = idx % a.nchunk;
    const int bg = idx / a.nchunk;
    const int b = bg / a.Hkv, g = bg % a.Hkv;

    // this lane's packed row: q head g*G + p / Nq, query row i = p % Nq
    const int p = rt * 32 + r32;
    const bool valid = p < a.rows_per_head;
    const int hq = g * a.G + (valid ? p / a.Nq : 0);
    const int i = valid ? p % a.Nq : 0;
    const long long grow = ((long long)b * a.Hq + hq) * a.Nq + i;  // row of out
    // the row's last allowed key (causal: bottom-right aligned)
    const int pos = CAUSAL && valid ? a.Nk - a.Nq + i : a.Nk - 1;

    const int nkb = (a.Nk + SAGE_BN - 1) / SAGE_BN;
    const int T0 = chunk * a.chunk_blocks;
    const int T1 = min(nkb, T0 + a.chunk_blocks);
    // blocks below this need no mask for any lane: no padding keys and no key
    // past the smallest causal limit (Nk - Nq)
    const int first_masked = CAUSAL ? min(a.Nk / SAGE_BN, (a.Nk - a.Nq + 1) / SAGE_BN) : a.Nk / SAGE_BN;

    const uint8_t* kbase = (const uint8_t*)a.k_i8 + (long long)bg * a.Np * D;
    const uint8_t* vbase = (const uint8_t*)a.v + (long long)bg * a.Np * D * VB;
    const float* ksc = a.k_scale + (long long)bg * (a.Np / (SAGE_BN / KSPLIT));

    v16f O[CT];
    float mref = -INFINITY, lsum = 0.0f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[ct][v] = 0.0f;

    // the query row and the first block's scales are loaded before the first
    // block's copy goes out (waits count in issue order), so the row is
    // quantized while the copy is in flight
    uint4 qraw[D / 16];
    load_q_row<D>(a.q + grow * D, valid, h, qraw);
    typedef float kvec __attribute__((ext_vector_type(KSPLIT)));
    kvec kscale = *reinterpret_cast<const kvec*>(ksc + KSPLIT * T0);
    typedef TileLoader<D, 1, VB> Loader;
    const Loader tiles(kbase, vbase, a.Np, 0, lane);
    tiles.load(T0, lk0, lv0, 0);
    // keep the quantization between the copy's issue and its wait: nothing
    // is scheduled across the barrier, and the empty asm statements take the
    // codes and scale as operands, so their computation cannot sink below
    // the wait
    __builtin_amdgcn_sched_barrier(0);
    v4i qf[D / 32];
    float sq = quantize_q_row<In, D>(qraw, qf);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) asm volatile("" : "+v"(qf[ks]));
    asm volatile("" : "+v"(sq));
    if constexpr (NBUF == 1) {
        // the first block's scores need its K tile only (the V tile was
        // issued after it, and waits count in issue order)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Loader::VR) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if constexpr (NBUF == 1) {
        // One buffer per tile: the next block's K tile is copied as soon as
        // this block's K fragments have been read, and its V tile once this
        // block's products have read theirs, so both copies run under this
        // block's work; each tile is waited for only where it is first read.
        for (int T = T0; T < T1; ++T) {
            const bool more = T + 1 < T1;
            const kvec knext = *reinterpret_cast<const kvec*>(ksc + KSPLIT * (more ? T + 1 : T));
            float c[KSPLIT];
#pragma unroll
            for (int gg = 0; gg < KSPLIT; ++gg) c[gg] = (sq * a.qk) * kscale[gg];
            v16i S[4];
            block_scores<D>(lk0, qf, h, r32, S);
            if (more) {
                // the K fragments are in registers: the tile can be replaced.
                // (The destination goes through an empty asm statement: with
                // its address in view, the compiler makes the V fragment reads
                // below wait for this copy; the explicit waits order them.)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                uint8_t* kdst = lk0;
                asm volatile("" : "+s"(kdst));
                tiles.load_k(T + 1, kdst, 0);
            }
            // V(T) was issued before knext and the next K tile
            if (more)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Loader::KR + 1) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
            if (T < first_masked)
                block_softmax_pv<D, KSPLIT, CAUSAL, PV16, false, V8>(
                    S, lv0, T, pos, a.Nk, c, a.l448, h, r32, rsel, mref, lsum, O);
            else
                block_softmax_pv<D, KSPLIT, CAUSAL, PV16, true, V8>(
                    S, lv0, T, pos, a.Nk, c, a.l448, h, r32, rsel, mref, lsum, O);
            kscale = knext;
            if (more) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                tiles.load_v(T + 1, lv0, 0);
                // the next block's scores need its K tile only
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Loader::VR) : "memory");
            }
        }
    }
    for (int T = T0; NBUF == 2 && T < T1; ++T) {
        const bool odd = NBUF == 2 && ((T - T0) & 1);
        const bool more = T + 1 < T1;
        // the next block's K scales before its tile copy (waits count in
        // issue order)
        const kvec knext = *reinterpret_cast<const kvec*>(ksc + KSPLIT * (more ? T + 1 : T));
        if (NBUF == 2 && more) tiles.load(T + 1, odd ? lk0 : lk1, odd ? lv0 : lv1, 0);
        float c[KSPLIT];
#pragma unroll
        for (int gg = 0; gg < KSPLIT; ++gg) c[gg] = (sq * a.qk) * kscale[gg];
        if (T < first_masked)
            attn_block<D, KSPLIT, CAUSAL, PV16, false, V8>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, pos,
                                                           a.Nk, c, a.l448, h, r32, rsel, mref, lsum, O);
        else
            attn_block<D, KSPLIT, CAUSAL, PV16, true, V8>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, pos,
                                                          a.Nk, c, a.l448, h, r32, rsel, mref, lsum, O);
        kscale = knext;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    if (!valid) return;
    // O[ct][v] is channel 32ct + 8(v/4) + 4h + v%4
    if (a.nchunk == 1) {
        const float* sv = a.v_scale + (long long)bg * D;
        const float inv_l = 1.0f / lsum;
        float* op = a.out + grow * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int ch = 32 * ct + 8 * k4 + 4 * h;
                const float4 s4 = *reinterpret_cast<const float4*>(sv + ch);
                float4 o;
                o.x = O[ct][4 * k4 + 0] * s4.x * inv_l;
                o.y = O[ct][4 * k4 + 1] * s4.y * inv_l;
                o.z = O[ct][4 * k4 + 2] * s4.z * inv_l;
                o.w = O[ct][4 * k4 + 3] * s4.w * inv_l;
                *reinterpret_cast<float4*>(op + ch) = o;
            }
        return;
    }
    const long long part = grow * a.nchunk + chunk;
    float* po = a.part_o + part * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const int ch = 32 * ct + 8 * k4 + 4 * h;
            const float4 o = {O[ct][4 * k4 + 0], O[ct][4 * k4 + 1], O[ct][4 * k4 + 2], O[ct][4 * k4 + 3]};
            *reinterpret_cast<float4*>(po + ch) = o;
        }
    if (h == 0) *reinterpret_cast<float2*>(a.part_ml + part * 2) = make_float2(mref, lsum);
}

// One work-group per (query row, 32 channels): out = O * s_V / l over the
// row's chunks, each weighted by 2^(its reference max - the largest).  Every
// thread issues its loads first (the max and row sum of chunks t, t + 256,
// ..., the partial O of its channel for chunks in its group, and the channel's
// V scale), so the merge waits on one round trip to memory; the largest max,
// the weighted row sum and the sum over chunk groups then take wave shuffles
// and one LDS exchange each.  Slicing the channels gives D / 32 work-groups
// per row, each with that fraction of the loads.  The key split never makes
// more than kMaxChunks chunks.  The arguments are plain scalars (not the
// DecodeArgs struct) so that the compiler can preload them into SGPRs.
constexpr int kMaxChunks = 1024;     // the most chunks a row may have
constexpr int kMergeSlice = 32;      // channels per merge work-group
constexpr int kMergeT = 256;         // threads per merge work-group
constexpr int kMergeLoads = 16;      // partial-O loads per thread issued together

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D>
__global__ __launch_bounds__(kMergeT) void decode_merge(const float* __restrict__ part_ml,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ v_scale,
                                                         float* __restrict__ out, int nchunk_,
                                                         int Nq, int Hq, int G, int Hkv) {
    constexpr int GROUPS = kMergeT / kMergeSlice;
    constexpr int NS = D / kMergeSlice;
    constexpr int MLU = kMaxChunks / kMergeT;
    __shared__ float wgt[kMaxChunks];
    __shared__ float osum[kMergeT];
    __shared__ float wmax[kMergeT / 64], wl[kMergeT / 64];
    const int row32 = blockIdx.x / NS, slice = blockIdx.x % NS;
    const long long row = row32;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nchunk = nchunk_;
    const int bh = row32 / Nq;
    const int hq = bh % Hq, b = bh / Hq;
    const int bg = b * Hkv + hq / G;
    const float* ml = part_ml + row * nchunk * 2;
    const float* po = part_o + row * nchunk * D;
    const int c = slice * kMergeSlice + (t % kMergeSlice), grp = t / kMergeSlice;
    const float vs = grp == 0 ? v_scale[(long long)bg * D + c] : 0.0f;

    float2 mlt[MLU];
#pragma unroll
    for (int u = 0; u < MLU; ++u) {
        const int k = t + u * kMergeT;
        mlt[u] = k < nchunk ? *reinterpret_cast<const float2*>(ml + 2 * k) : make_float2(-INFINITY, 0.0f);
    }
    float x[kMergeLoads];
#pragma unroll
    for (int u = 0; u < kMergeLoads; ++u) {
        const int k = grp + u * GROUPS;
        x[u] = k < nchunk ? po[(long long)k * D + c] : 0.0f;
    }
    float m = mlt[0].x;
#pragma unroll
    for (int u = 1; u < MLU; ++u) m = fmaxf(m, mlt[u].x);
    const float mw = wave_max(m);
    if (lane == 0) wmax[wave] = mw;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int i = 1; i < kMergeT / 64; ++i) M = fmaxf(M, wmax[i]);
    float lt = 0.0f;
#pragma unroll
    for (int u = 0; u < MLU; ++u) {
        const int k = t + u * kMergeT;
        const float w = k < nchunk ? __builtin_amdgcn_exp2f(mlt[u].x - M) : 0.0f;
        wgt[k] = w;
        lt = __builtin_fmaf(mlt[u].y, w, lt);
    }
    const float lw = wave_sum(lt);
    if (lane == 0) wl[wave] = lw;
    __syncthreads();
    float l = 0.0f;
#pragma unroll
    for (int i = 0; i < kMergeT / 64; ++i) l += wl[i];

    float o = 0.0f;
#pragma unroll
    for (int u = 0; u < kMergeLoads; ++u) {
        const int k = grp + u * GROUPS;
        if (k < nchunk) o = __builtin_fmaf(x[u], wgt[k], o);
    }
    for (int k = grp + kMergeLoads * GROUPS; k < nchunk; k += GROUPS)
        o = __builtin_fmaf(po[(long long)k * D + c], wgt[k], o);
    osum[t] = o;
    __syncthreads();
    if (grp == 0) {
#pragma unroll
        for (int g2 = 1; g2 < GROUPS; ++g2) o += osum[g2 * kMergeSlice + (t % kMergeSlice)];
        out[row * D + c] = o * vs * (1.0f / l);
    }
}

#define SAGE_DECODE_INST(In, D, KSPLIT, CAUSAL, PV16) \
    template __global__ void attn_decode<In, D, KSPLIT, CAUSAL, PV16>(DecodeArgs);
#define SAGE_DECODE_INST_PV(In, D, KSPLIT, CAUSAL) \
    SAGE_DECODE_INST(In, D, KSPLIT, CAUSAL, false) SAGE_DECODE_INST(In, D, KSPLIT, CAUSAL, true)
#define SAGE_DECODE_INST_C(In, D, KSPLIT) \
    SAGE_DECODE_INST_PV(In, D, KSPLIT, false) SAGE_DECODE_INST_PV(In, D, KSPLIT, true)
#define SAGE_DECODE_INST_K(In, D) SAGE_DECODE_INST_C(In, D, 2) SAGE_DECODE_INST_C(In, D, 4)
SAGE_DECODE_INST_K(_Float16, 64)
SAGE_DECODE_INST_K(_Float16, 128)
SAGE_DECODE_INST_K(Bf16Tag, 64)
SAGE_DECODE_INST_K(Bf16Tag, 128)
#undef SAGE_DECODE_INST_K
#undef SAGE_DECODE_INST_C
#undef SAGE_DECODE_INST_PV
#undef SAGE_DECODE_INST
template __global__ void decode_merge<64>(const float*, const float*, const float*, float*, int, int, int, int, int);
template __global__ void decode_merge<128>(const float*, const float*, const float*, float*, int, int, int, int, int);

// Chunking: about one round of work-groups, wgs_per_cu per CU, in chunks of
// at least kMinChunkBlocks blocks so that filling each work-group's tile
// pipeline stays a small part of its work.  One round beat two on both the
// 32768-key single-sequence cache and the batch of eight 8192-key caches
// (fewer partials to merge, no second-round tail).  The chunk count rounds
// down so that the grid does not spill a short second round.
constexpr int kMinChunkBlocks = 2;
static_assert(256 * kDecodeWavesPerCU <= kMaxChunks, "a row's chunks must fit the merge's weight table");

DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int wgs_per_cu) {
    DecodePlan pl;
    const int G = Hq / Hkv;
    pl.row_tiles = (G * Nq + 31) / 32;
    const int nkb = (Nk + SAGE_BN - 1) / SAGE_BN;
    const long long units = (long long)B * Hkv * pl.row_tiles;
    (void)d;
    const long long target = 256LL * wgs_per_cu;
    long long want = target / units;
    if (want < 1) want = 1;
    int per = (int)((nkb + want - 1) / want);
    if (per < kMinChunkBlocks) per = kMinChunkBlocks;
    if (per > nkb) per = nkb;
    pl.chunk_blocks = per;
    pl.nchunk = (nkb + per - 1) / per;
    return pl;
}

template <typename In, int D, int KSPLIT, bool CAUSAL, bool PV16>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    constexpr size_t lds = decode_lds<D, PV16>();
    if (a.nchunk > kMaxChunks) return hipErrorInvalidValue;  // not reached: see decode_plan
    if (lds > 65536) {
        static LaunchFacts facts;
        int slots = 0;
        hipError_t e = facts.settle((const void*)attn_decode<In, D, KSPLIT, CAUSAL, PV16>, 64, lds, &slots);
        if (e != hipSuccess) return e;
    }
    const long long grid = (long long)a.B * a.Hkv * a.nchunk * a.row_tiles;
    hipLaunchKernelGGL((attn_decode<In, D, KSPLIT, CAUSAL, PV16>), dim3((unsigned)grid), dim3(64), lds,
                       st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nchunk == 1) return e;
    hipLaunchKernelGGL((decode_merge<D>), dim3((unsigned)((long long)a.B * a.Hq * a.Nq * (D / kMergeSlice))),
                       dim3(kMergeT), 0, st, a.part_ml, a.part_o, a.v_scale, a.out, a.nchunk, a.Nq, a.Hq,
                       a.G, a.Hkv);
    return hipGetLastError();
}

template <typename In, int D, int KSPLIT>
static hipError_t launch_decode_k(const DecodeArgs& a, int causal, bool pv16, hipStream_t st) {
    if (causal)
        return pv16 ? launch_decode_t<In, D, KSPLIT, true, true>(a, st)
                    : launch_decode_t<In, D, KSPLIT, true, false>(a, st);
    return pv16 ? launch_decode_t<In, D, KSPLIT, false, true>(a, st)
                : launch_decode_t<In, D, KSPLIT, false, false>(a, st);
}

template <typename In, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, bool fine_k, int causal, bool pv16,
                                  hipStream_t st) {
    return fine_k ? launch_decode_k<In, D, 4>(a, causal, pv16, st)
                  : launch_decode_k<In, D, 2>(a, causal, pv16, st);
}

hipError_t launch_decode(const void* q, int dtype, const sage_kv_cache* cache, float* out,
                         float* part_o, float* part_ml, int B, int Hq, int Hkv, int Nq, int Nk,
                         int d, int causal, float qk, float l448, hipStream_t st) {
    const bool pv16 = cache->pv_format == SAGE_PV_F16;
    const int wpc = d == 64 ? (pv16 ? decode_wgs_per_cu<64, true>() : decode_wgs_per_cu<64, false>())
                            : (pv16 ? decode_wgs_per_cu<128, true>() : decode_wgs_per_cu<128, false>());
    const DecodePlan pl = decode_plan(B, Hq, Hkv, Nq, Nk, d, wpc);
    DecodeArgs a;
    a.q = (const uint16_t*)q;
    a.k_i8 = cache->k_i8;
    a.k_scale = cache->k_scale;
    a.v = cache->v;
    a.v_scale = cache->v_scale;
    a.out = out;
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Nq = Nq;
    a.Nk = Nk;
    a.Np = make_shape(B, Hq, Hkv, Nk, d).Np;
    a.G = Hq / Hkv;
    a.rows_per_head = a.G * Nq;
    a.row_tiles = pl.row_tiles;
    a.nchunk = pl.nchunk;
    a.chunk_blocks = pl.chunk_blocks;
    a.qk = qk;
    a.l448 = l448;
    const bool fine_k = cache->k_block == SAGE_BK_THREAD;
    if (dtype == SAGE_F16)
        return d == 64 ? launch_decode_d<_Float16, 64>(a, fine_k, causal, pv16, st)
                       : launch_decode_d<_Float16, 128>(a, fine_k, causal, pv16, st);
    return d == 64 ? launch_decode_d<Bf16Tag, 64>(a, fine_k, causal, pv16, st)
                   : launch_decode_d<Bf16Tag, 128>(a, fine_k, causal, pv16, st);
}

}  // namespace sage
