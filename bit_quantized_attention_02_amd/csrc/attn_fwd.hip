// Fused 8-bit attention forward (prefill) for CDNA4 (gfx950).
//
// One work-group = WAVES waves = 32*WAVES query rows of one (batch, q head);
// each wave owns 32 rows, one 32-wide matrix-core tile, and loops over the
// key blocks with the per-block computation of attn_block.h (double-buffered
// LDS tiles, INT8 Q.K^T, FP32 online softmax, E4M3 or binary16 P, two-level
// P.V).
#include <type_traits>

#include "attn_block.h"

namespace sage {

static_assert(SAGE_BQ == 128 && SAGE_BQ_THREAD == 1 && SAGE_BK == 64 && SAGE_BK_THREAD == 32 &&
                  SAGE_BK_TOKEN == 1,
              "the launch maps the granularities to q_shift 7/0 and 2/4/128 K scales per block");

constexpr int kMaxTailSplit = 8;  // key shares of a split tail tile, at most

struct AttnArgs {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint16_t* v16;
    const float* v_scale;
    float* out;
    int B, Hq, Hkv, N, Np, G, nqt;
    // The last partial round's tiles, when split along the keys: tiles
    // [tiles_main, B*Hq*nqt) each take tail_split work-groups, whose partial
    // results (unnormalised O [.., D] in part_o, reference max and row sum in
    // part_ml) attn_tail_merge combines.  tiles_main = B*Hq*nqt: no split.
    int tiles_main, tail_split;
    float* part_o;
    float* part_ml;
    long long tail_rows;  // rows part_o / part_ml hold (0: no split)
    int q_shift;  // log2 of the query rows per Q scale (7 or 0)
    float qk;    // f32(sm_scale * log2 e)
    float l448;  // f32(log2 448), or 0 for binary16 P
};

template <int D, int KSPLIT, bool CAUSAL, bool PV16, int WAVES, int WAVES_PER_SIMD>
__global__ __launch_bounds__(64 * WAVES, WAVES_PER_SIMD) void attn_fwd(AttnArgs a) {
    constexpr int KS = D / 32;
    constexpr int CT = D / 32;
    constexpr int ROWS = 32 * WAVES;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* const lk0 = smem;
    uint8_t* const lk1 = smem + SAGE_BN * D;
    uint16_t* const lv0 = reinterpret_cast<uint16_t*>(smem + 2 * SAGE_BN * D);
    uint16_t* const lv1 = lv0 + D * SAGE_BN;
    // with one K scale per key, each block's 128 scales ride with its tiles
    constexpr bool PER_KEY = KSPLIT == SAGE_BN;
    float* const ls0 = reinterpret_cast<float*>(lv1 + D * SAGE_BN);
    float* const ls1 = ls0 + SAGE_BN;

    const int lane = threadIdx.x & 63;
    // The wave index is uniform; held in a scalar register at d = 64, the
    // tile copies' LDS addresses are formed without vector instructions.  (At
    // d = 128 the scalar form makes the compiler spill registers in the
    // causal loops.)
    const int wave = D == 64 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
    const int h = lane >> 5, r32 = lane & 31;
    const v8h rsel = row_sum_selector(lane);

    // Work-group -> tile.  Work-groups are dispatched round-robin over the 8
    // XCDs; give each XCD a contiguous range of tiles (same heads, so K and V
    // stay in that XCD's L2).
    // A split tail tile's work-groups come after all the others.
    const int main_tiles = a.tiles_main;
    int logical, chunk = -1;
    if ((int)blockIdx.x < main_tiles) {
        const int per_xcd = (main_tiles + 7) / 8;
        const int tall = main_tiles % 8 == 0 ? 8 : main_tiles % 8;
        const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
        const int start = xcd < tall ? xcd * per_xcd : tall * per_xcd + (xcd - tall) * (per_xcd - 1);
        const int count = xcd < tall ? per_xcd : per_xcd - 1;
        logical = start + local;
        // causal: when an XCD's range holds whole heads, go through it by
        // tile length (each head's longest tile, then the next longest, ...)
        // so that no long tile starts late
        if (CAUSAL && start % a.nqt == 0 && count % a.nqt == 0) {
            const int heads = count / a.nqt;
            logical = start + (local % heads) * a.nqt + local / heads;
        }
    } else {
        const int j = blockIdx.x - main_tiles;
        logical = main_tiles + j / a.tail_split;
        chunk = j % a.tail_split;
    }
    const int qt_l = logical % a.nqt;
    const int bh = logical / a.nqt;
    const int hq = bh % a.Hq, b = bh / a.Hq;
    const int qt = CAUSAL ? a.nqt - 1 - qt_l : qt_l;  // causal: longest rows first
    const int bg = b * a.Hkv + hq / a.G;
    const int q0 = qt * ROWS;
    const int rbase = q0 + 32 * wave;  // this wave's first row
    const int row = rbase + r32;       // this lane's row

    const int nkb = (a.N + SAGE_BN - 1) / SAGE_BN;  // key blocks holding real keys
    const int nblk = CAUSAL ? min(nkb, (q0 + ROWS - 1) / SAGE_BN + 1) : nkb;
    // blocks [0, n_full) need no mask for any row of this wave; the wave
    // stops after wave_last
    const int n_full = CAUSAL ? min(rbase / SAGE_BN, a.N / SAGE_BN) : a.N / SAGE_BN;
    const int wave_last = CAUSAL ? min(nkb - 1, (rbase + 31) / SAGE_BN) : nkb - 1;

    // key blocks [T0, T1): all of them, or a split tile's share (non-causal)
    int T0 = 0, T1 = nblk;
    if (chunk >= 0) {
        T0 = (int)((long long)chunk * nblk / a.tail_split);
        T1 = (int)((long long)(chunk + 1) * nblk / a.tail_split);
    }

    const uint8_t* kbase = (const uint8_t*)a.k_i8 + (long long)bg * a.Np * D;
    const uint16_t* vbase = a.v16 + (long long)bg * a.Np * D;
    const float* ksc = a.k_scale + (long long)bg * (a.Np / (SAGE_BN / KSPLIT));

    // Q fragments (B operand of Q.K^T): query row r32, bytes [32*ks + 16*h, +16).
    v4i qf[KS];
    {
        const int8_t* qp = a.q_i8 + ((long long)bh * a.Np + row) * D + 16 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const v4i*>(qp + 32 * ks);
    }
    // this lane's Q scale (its row's block, or its own row)
    const float sq = a.q_scale[(long long)bh * (a.Np >> a.q_shift) + (row >> a.q_shift)];

    v16f O[CT];
    float mref = -INFINITY, lsum = 0.0f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[ct][v] = 0.0f;

    // The K scales of a block are loaded one block ahead, before that block's
    // tile copy is issued: vector-memory waits count in issue order, so a
    // scale load issued after the copy would make its wait cover the copy too.
    // (per key the scales go through LDS instead; see load_s)
    constexpr int NKS = PER_KEY ? 1 : KSPLIT;
    typedef float kvec __attribute__((ext_vector_type(NKS)));
    auto load_kscale = [&](int t) -> kvec {
        if constexpr (PER_KEY) {
            (void)t;
            return kvec{};
        } else {
            return *reinterpret_cast<const kvec*>(ksc + KSPLIT * t);
        }
    };
    kvec kscale = load_kscale(T0);
    const TileLoader<D, WAVES> tiles(kbase, vbase, a.Np, wave, lane);
    // the 128 per-key scales of block t into LDS: one float per lane of the
    // first two waves, written straight to LDS by the buffer load
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void*)ksc, (short)0, PER_KEY ? a.Np * 4 : 0, 0x00020000);
    auto load_s = [&](int t, float* ls) {
        if (PER_KEY && wave < 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                srs, (__attribute__((address_space(3))) void*)(ls + 64 * wave), 4, lane * 4,
                t * SAGE_BN * 4 + wave * 256, 0, 0);
    };
    // the score factors of a block (see score_factors)
    auto factors = [&](float (&c)[score_factors<KSPLIT>()]) {
        const float sqq = sq * a.qk;  // the row's part of every factor
        if constexpr (PER_KEY) {
            c[0] = sqq;
        } else {
#pragma unroll
            for (int g = 0; g < KSPLIT; ++g) c[g] = sqq * kscale[g];
        }
    };
    tiles.load(T0, lk0, lv0, wave);
    load_s(T0, ls0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Blocks [0, nA) need no mask for any wave of the work-group: a loop of
    // its own keeps that body free of per-wave branches.
    const int nA = CAUSAL ? min(q0 / SAGE_BN, a.N / SAGE_BN) : a.N / SAGE_BN;
    // At d = 64 that loop goes two blocks at a time, so that each copy of
    // the body reads and fills fixed buffers (their LDS offsets become
    // immediates; at d = 128 the second copy would push registers into
    // spills).
    // (Buffers alternate with the block's place after T0.)
    auto full_block = [&](int T, auto odd_c) {
        constexpr bool ODD = decltype(odd_c)::value;
        const bool more = T + 1 < T1;
        const kvec knext = load_kscale(more ? T + 1 : T);
        if (more) {
            tiles.load(T + 1, ODD ? lk0 : lk1, ODD ? lv0 : lv1, wave);
            load_s(T + 1, ODD ? ls0 : ls1);
        }
        float c[score_factors<KSPLIT>()];
        factors(c);
        attn_block<D, KSPLIT, CAUSAL, PV16, false>(ODD ? lk1 : lk0, ODD ? lv1 : lv0, qf, T, row, a.N, c, a.l448,
                                                   h, r32, rsel, mref, lsum, O, ODD ? ls1 : ls0);
        kscale = knext;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    typedef std::integral_constant<bool, false> even_t;
    typedef std::integral_constant<bool, true> odd_t;
    const int nA1 = min(nA, T1);
    int T = T0;
    if constexpr (D == 64) {
        for (; T + 1 < nA1; T += 2) {
            full_block(T, even_t());
            full_block(T + 1, odd_t());
        }
        if (T < nA1) full_block(T++, even_t());  // T - T0 is even here
    } else {
        for (; T < nA1; ++T) {
            const bool odd = (T - T0) & 1;
            const bool more = T + 1 < T1;
            const kvec knext = load_kscale(more ? T + 1 : T);
            if (more) {
                tiles.load(T + 1, odd ? lk0 : lk1, odd ? lv0 : lv1, wave);
                load_s(T + 1, odd ? ls0 : ls1);
            }
            float c[score_factors<KSPLIT>()];
            factors(c);
            attn_block<D, KSPLIT, CAUSAL, PV16, false>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, row, a.N, c,
                                                       a.l448, h, r32, rsel, mref, lsum, O, odd ? ls1 : ls0);
            kscale = knext;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
    for (; T < T1; ++T) {
        const bool odd = (T - T0) & 1;
        const bool more = T + 1 < T1;
        const kvec knext = load_kscale(more ? T + 1 : T);
        if (more) {
            tiles.load(T + 1, odd ? lk0 : lk1, odd ? lv0 : lv1, wave);
            load_s(T + 1, odd ? ls0 : ls1);
        }
        float c[score_factors<KSPLIT>()];
        factors(c);
        // (without causality only the ragged last block is left here: one
        // body, whose registers then need no spilling at d = 128)
        if (CAUSAL && T < n_full)
            attn_block<D, KSPLIT, CAUSAL, PV16, false>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, row, a.N, c,
                                                       a.l448, h, r32, rsel, mref, lsum, O, odd ? ls1 : ls0);
        else if (T <= wave_last)
            attn_block<D, KSPLIT, CAUSAL, PV16, true>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, row, a.N, c,
                                                      a.l448, h, r32, rsel, mref, lsum, O, odd ? ls1 : ls0);
        kscale = knext;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: out = O * s_V / l.  O[ct][v] is channel 32ct + 8(v/4) + 4h + v%4.
    if (chunk >= 0) {
        if (row >= a.N) return;
        // a split tile's share: unnormalised O, reference max, row sum
        const long long p = ((long long)(logical - main_tiles) * ROWS + (row - q0)) * a.tail_split + chunk;
        float* po = a.part_o + p * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 32 * ct + 8 * i + 4 * h;
                const float4 o = {O[ct][4 * i + 0], O[ct][4 * i + 1], O[ct][4 * i + 2], O[ct][4 * i + 3]};
                *reinterpret_cast<float4*>(po + ch) = o;
            }
        if (h == 0) *reinterpret_cast<float2*>(a.part_ml + p * 2) = make_float2(mref, lsum);
        return;
    }
    const float* sv = a.v_scale + (long long)bg * D;
    const float inv_l = 1.0f / lsum;
    if constexpr (D == 64) {
        // each lane stores its row's values directly (turning them around
        // through LDS as below costs the block loop registers at d = 64,
        // whose long tiles make the epilogue a small part of the time)
        if (row >= a.N) return;
        float* op = a.out + ((long long)bh * a.N + row) * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 32 * ct + 8 * i + 4 * h;
                const float4 s4 = *reinterpret_cast<const float4*>(sv + ch);
                float4 o;
                o.x = O[ct][4 * i + 0] * s4.x * inv_l;
                o.y = O[ct][4 * i + 1] * s4.y * inv_l;
                o.z = O[ct][4 * i + 2] * s4.z * inv_l;
                o.w = O[ct][4 * i + 3] * s4.w * inv_l;
                *reinterpret_cast<float4*>(op + ch) = o;
            }
        return;
    }
    // d = 128: each wave turns its 32 rows around through an LDS region of
    // its own (the tile buffers are free after the last block's barrier), 64
    // channels at a time, so that each store instruction writes whole rows'
    // 256-byte runs instead of a lane's scattered 16-byte pieces: the short
    // causal tiles end sooner.  Rows are padded to 68 floats, so the 16
    // lanes of a 16-byte write phase land on distinct banks.
    constexpr int RS = 68;
    float* const lo = reinterpret_cast<float*>(smem) + wave * 32 * RS;
    float* const ob = a.out + (long long)bh * a.N * D;
#pragma unroll
    for (int pass = 0; pass < CT / 2; ++pass) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ct = 2 * pass + cc;
                const int ch = 32 * ct + 8 * i + 4 * h;
                const float4 s4 = *reinterpret_cast<const float4*>(sv + ch);
                float4 o;
                o.x = O[ct][4 * i + 0] * s4.x * inv_l;
                o.y = O[ct][4 * i + 1] * s4.y * inv_l;
                o.z = O[ct][4 * i + 2] * s4.z * inv_l;
                o.w = O[ct][4 * i + 3] * s4.w * inv_l;
                *reinterpret_cast<float4*>(lo + r32 * RS + ch - 64 * pass) = o;
            }
        // (a wave's LDS accesses run in order: these reads see the writes
        // above, and the next pass's writes come after them)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = lane + 64 * k, rr = c >> 4, c4 = c & 15;
            const float4 o = *reinterpret_cast<const float4*>(lo + rr * RS + 4 * c4);
            if (rbase + rr < a.N)
                *reinterpret_cast<float4*>(ob + (long long)(rbase + rr) * D + 64 * pass + 4 * c4) = o;
        }
    }
}

// d = 64: 4-wave work-groups (48 KB of LDS each) whose waves interleave on
// each SIMD: three per CU (168 registers a wave) for the non-causal
// per-block and thread-level granularities, whose loops fit those registers
// (the thread-level one reloads two spilled registers per block); two per CU
// (half the register file) otherwise.  d = 128: one 8-wave work-group per CU
// (96 KB of LDS), two waves per SIMD.
template <int D>
constexpr int attn_waves() {
    return D == 64 ? 4 : 8;
}
template <int D, int KSPLIT, bool CAUSAL>
constexpr int attn_waves_per_simd() {
    return D == 64 && (KSPLIT == 2 || KSPLIT == 4) && !CAUSAL ? 3 : 2;
}

// Combines the key-split shares of the last partial round's tiles: per query
// row, out = sum_c 2^(m_c - M) O_c * s_V / sum_c 2^(m_c - M) l_c with M the
// largest reference max of the row's shares.  One thread per (row, four
// channels): 16-byte loads of each share's partial output.
template <int D>
__global__ __launch_bounds__(256) void attn_tail_merge(AttnArgs a, int rows_per_tile) {
    constexpr int C4 = D / 4;
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const int ch = 4 * (int)(gid % C4);
    const long long rr = gid / C4;  // row among the split tiles' rows
    const long long tail_rows = (long long)(a.B * a.Hq * a.nqt - a.tiles_main) * rows_per_tile;
    if (rr >= tail_rows) return;
    const int logical = a.tiles_main + (int)(rr / rows_per_tile);
    const int row = (logical % a.nqt) * rows_per_tile + (int)(rr % rows_per_tile);
    if (row >= a.N) return;
    const int bh = logical / a.nqt;
    const int hq = bh % a.Hq, b = bh / a.Hq;
    const int bg = b * a.Hkv + hq / a.G;
    const int S = a.tail_split;
    const float* ml = a.part_ml + rr * S * 2;
    const float* po = a.part_o + rr * S * D + ch;
    float M = ml[0];
    for (int c = 1; c < S; ++c) M = fmaxf(M, ml[2 * c]);
    float l = 0.0f;
    float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < S; ++c) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * c] - M);
        const float4 x = *reinterpret_cast<const float4*>(po + (long long)c * D);
        l = __builtin_fmaf(ml[2 * c + 1], w, l);
        o.x = __builtin_fmaf(x.x, w, o.x);
        o.y = __builtin_fmaf(x.y, w, o.y);
        o.z = __builtin_fmaf(x.z, w, o.z);
        o.w = __builtin_fmaf(x.w, w, o.w);
    }
    const float4 sv = *reinterpret_cast<const float4*>(a.v_scale + (long long)bg * D + ch);
    const float inv_l = 1.0f / l;
    float4 r;
    r.x = o.x * sv.x * inv_l;
    r.y = o.y * sv.y * inv_l;
    r.z = o.z * sv.z * inv_l;
    r.w = o.w * sv.w * inv_l;
    *reinterpret_cast<float4*>(a.out + ((long long)bh * a.N + row) * D + ch) = r;
}
template __global__ void attn_tail_merge<64>(AttnArgs, int);
template __global__ void attn_tail_merge<128>(AttnArgs, int);

// Explicit instantiations: with the packed-FP32 feature switched off on the
// command line, this compiler otherwise leaves the host stubs of some of these
// kernels undefined.
#define SAGE_ATTN_INST(D, KSPLIT, CAUSAL, PV16)                                                   \
    template __global__ void                                                                        \
    attn_fwd<D, KSPLIT, CAUSAL, PV16, attn_waves<D>(), attn_waves_per_simd<D, KSPLIT, CAUSAL>()>(AttnArgs);
#define SAGE_ATTN_INST_PV(D, KSPLIT, CAUSAL) \
    SAGE_ATTN_INST(D, KSPLIT, CAUSAL, false) SAGE_ATTN_INST(D, KSPLIT, CAUSAL, true)
SAGE_ATTN_INST_PV(64, 2, false)
SAGE_ATTN_INST_PV(64, 2, true)
SAGE_ATTN_INST_PV(64, 4, false)
SAGE_ATTN_INST_PV(64, 4, true)
SAGE_ATTN_INST_PV(128, 2, false)
SAGE_ATTN_INST_PV(128, 2, true)
SAGE_ATTN_INST_PV(128, 4, false)
SAGE_ATTN_INST_PV(128, 4, true)
SAGE_ATTN_INST_PV(64, SAGE_BN, false)
SAGE_ATTN_INST_PV(64, SAGE_BN, true)
SAGE_ATTN_INST_PV(128, SAGE_BN, false)
SAGE_ATTN_INST_PV(128, SAGE_BN, true)
#undef SAGE_ATTN_INST_PV
#undef SAGE_ATTN_INST

template <int D, int KSPLIT, bool CAUSAL, bool PV16>
static hipError_t launch_attn_t(AttnArgs a, hipStream_t st) {
    constexpr int WAVES = attn_waves<D>();
    constexpr int WPS = attn_waves_per_simd<D, KSPLIT, CAUSAL>();
    constexpr size_t lds = 2 * SAGE_BN * D + 2 * D * SAGE_BN * 2 + (KSPLIT == SAGE_BN ? 2 * SAGE_BN * 4 : 0);
    a.nqt = a.Np / (32 * WAVES);
    const void* fn = (const void*)attn_fwd<D, KSPLIT, CAUSAL, PV16, WAVES, WPS>;
    static LaunchFacts facts;
    int slots = 0;
    {
        hipError_t e = facts.settle(fn, 64 * WAVES, lds, &slots);
        if (e != hipSuccess) return e;
    }
    const int total = a.B * a.Hq * a.nqt;
    constexpr int ROWS = 32 * WAVES;
    // The last partial round: when the tiles do not fill whole rounds of the
    // work-groups the chip runs at once, the leftover tiles (non-causal, all
    // equally long) are split along the keys over the otherwise idle slots.
    a.tiles_main = total;
    a.tail_split = 1;
    if (!CAUSAL && a.part_o != nullptr && slots > 0) {
        const int nkb = (a.N + SAGE_BN - 1) / SAGE_BN;
        const int tail = total > slots ? total % slots : 0;
        if (tail > 0) {
            // The leftover tiles as `split` shares each run in
            // ceil(tail * split / slots) waves of 1/split of a tile's
            // time: take the split with the shortest, if it beats the
            // whole tiles' one wave, within the partials' room.
            int best = 1;
            long long best_num = 1, best_den = 1;  // time as a fraction of a tile's
            for (int split = 2; split <= kMaxTailSplit && split <= nkb; ++split) {
                if ((long long)tail * split * ROWS > a.tail_rows) break;
                const long long waves = ((long long)tail * split + slots - 1) / slots;
                if (waves * best_den < best_num * split) {
                    best = split;
                    best_num = waves;
                    best_den = split;
                }
            }
            if (best > 1) {
                a.tiles_main = total - tail;
                a.tail_split = best;
            }
        }
    }
    const int grid = a.tiles_main + (total - a.tiles_main) * a.tail_split;
    hipLaunchKernelGGL((attn_fwd<D, KSPLIT, CAUSAL, PV16, WAVES, WPS>), dim3(grid), dim3(64 * WAVES), lds,
                       st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.tail_split == 1) return e;
    const long long threads = (long long)(total - a.tiles_main) * ROWS * (D / 4);
    hipLaunchKernelGGL((attn_tail_merge<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a,
                       ROWS);
    return hipGetLastError();
}

template <int D, int KSPLIT, bool PV16>
static hipError_t launch_attn_p(AttnArgs a, int causal, hipStream_t st) {
    return causal ? launch_attn_t<D, KSPLIT, true, PV16>(a, st) : launch_attn_t<D, KSPLIT, false, PV16>(a, st);
}

template <int D, int KSPLIT>
static hipError_t launch_attn_d(AttnArgs a, int causal, bool pv16, hipStream_t st) {
    return pv16 ? launch_attn_p<D, KSPLIT, true>(a, causal, st) : launch_attn_p<D, KSPLIT, false>(a, causal, st);
}

hipError_t launch_attn(const sage_qkv_quant* z, float* out, const Shape& s, int causal,
                       float qk, float l448, hipStream_t st) {
    AttnArgs a;
    a.q_i8 = z->q_i8;
    a.q_scale = z->q_scale;
    a.k_i8 = z->k_i8;
    a.k_scale = z->k_scale;
    a.v16 = z->v16;
    a.v_scale = z->v_scale;
    a.out = out;
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.Np = s.Np;
    a.G = s.Hq / s.Hkv;
    a.nqt = 0;
    a.tiles_main = 0;
    a.tail_split = 1;
    a.tail_rows = z->tail_part ? z->tail_rows : 0;
    a.part_o = a.tail_rows > 0 ? z->tail_part : nullptr;
    a.part_ml = a.tail_rows > 0 ? z->tail_part + a.tail_rows * s.d : nullptr;
    a.q_shift = z->q_block == SAGE_BQ ? 7 : 0;  // SAGE_BQ = 128, SAGE_BQ_THREAD = 1
    a.qk = qk;
    a.l448 = l448;
    // K scales per block: 2 (SAGE_BK), 4 (SAGE_BK_THREAD) or one per key (SAGE_BK_TOKEN)
    const bool pv16 = z->pv_format == SAGE_PV_F16;
    // (INT4 codes go through the same kernels: their scores are as exact)
    if (s.d == 64) {
        if (z->k_block == SAGE_BK_TOKEN) return launch_attn_d<64, SAGE_BN>(a, causal, pv16, st);
        return z->k_block == SAGE_BK_THREAD ? launch_attn_d<64, 4>(a, causal, pv16, st)
                                            : launch_attn_d<64, 2>(a, causal, pv16, st);
    }
    if (z->k_block == SAGE_BK_TOKEN) return launch_attn_d<128, SAGE_BN>(a, causal, pv16, st);
    return z->k_block == SAGE_BK_THREAD ? launch_attn_d<128, 4>(a, causal, pv16, st)
                                        : launch_attn_d<128, 2>(a, causal, pv16, st);
}

}  // namespace sage
