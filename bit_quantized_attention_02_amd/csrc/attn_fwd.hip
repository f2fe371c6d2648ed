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

static_assert(SAGE_BQ == 128 && SAGE_BQ_THREAD == 1 && SAGE_BK == 64 && SAGE_BK_THREAD == 32,
              "the launch maps the two granularities to q_shift 7/0 and 2/4 K scales per block");

struct AttnArgs {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint16_t* v16;
    const float* v_scale;
    float* out;
    int B, Hq, Hkv, N, Np, G, nqt;
    int q_shift;  // log2 of the query rows per Q scale (7 or 0)
    float qk;    // f32(sm_scale * log2 e)
    float l448;  // f32(log2 448), or 0 for binary16 P
};

template <int D, int KSPLIT, bool CAUSAL, bool PV16, bool SEEDED, int WAVES, int WAVES_PER_SIMD>
__global__ __launch_bounds__(64 * WAVES, WAVES_PER_SIMD) void attn_fwd(AttnArgs a) {
    constexpr int KS = D / 32;
    constexpr int CT = D / 32;
    constexpr int ROWS = 32 * WAVES;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* const lk0 = smem;
    uint8_t* const lk1 = smem + SAGE_BN * D;
    uint16_t* const lv0 = reinterpret_cast<uint16_t*>(smem + 2 * SAGE_BN * D);
    uint16_t* const lv1 = lv0 + D * SAGE_BN;

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
    const int total = a.B * a.Hq * a.nqt;
    const int per_xcd = (total + 7) / 8;
    const int tall = total % 8 == 0 ? 8 : total % 8;
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const int logical = xcd < tall ? xcd * per_xcd + local
                                   : tall * per_xcd + (xcd - tall) * (per_xcd - 1) + local;
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
    typedef float kvec __attribute__((ext_vector_type(KSPLIT)));
    kvec kscale = *reinterpret_cast<const kvec*>(ksc);
    const TileLoader<D, WAVES> tiles(kbase, vbase, a.Np, wave, lane);
    tiles.load(0, lk0, lv0, wave);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Blocks [0, nA) need no mask for any wave of the work-group: a loop of
    // its own keeps that body free of per-wave branches.
    const int nA = CAUSAL ? min(q0 / SAGE_BN, a.N / SAGE_BN) : a.N / SAGE_BN;
    // At d = 64 that loop goes two blocks at a time, so that each copy of
    // the body reads and fills fixed buffers (their LDS offsets become
    // immediates; at d = 128 the second copy would push registers into
    // spills).
    auto full_block = [&](int T, auto odd_c) {
        constexpr bool ODD = decltype(odd_c)::value;
        const bool more = T + 1 < nblk;
        const kvec knext = *reinterpret_cast<const kvec*>(ksc + KSPLIT * (more ? T + 1 : T));
        if (more) tiles.load(T + 1, ODD ? lk0 : lk1, ODD ? lv0 : lv1, wave);
        float c[KSPLIT];
#pragma unroll
        for (int g = 0; g < KSPLIT; ++g) c[g] = (sq * kscale[g]) * a.qk;
        attn_block<D, KSPLIT, CAUSAL, PV16, false, false, SEEDED>(ODD ? lk1 : lk0, ODD ? lv1 : lv0, qf, T, row,
                                                                 a.N, c, a.l448, h, r32, rsel, mref, lsum, O);
        kscale = knext;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    typedef std::integral_constant<bool, false> even_t;
    typedef std::integral_constant<bool, true> odd_t;
    int T = 0;
    if constexpr (D == 64) {
        for (; T + 1 < nA; T += 2) {
            full_block(T, even_t());
            full_block(T + 1, odd_t());
        }
        if (T < nA) full_block(T++, even_t());  // T is even here
    } else {
        for (; T < nA; ++T) {
            const bool odd = T & 1;
            const bool more = T + 1 < nblk;
            const kvec knext = *reinterpret_cast<const kvec*>(ksc + KSPLIT * (more ? T + 1 : T));
            if (more) tiles.load(T + 1, odd ? lk0 : lk1, odd ? lv0 : lv1, wave);
            float c[KSPLIT];
#pragma unroll
            for (int g = 0; g < KSPLIT; ++g) c[g] = (sq * kscale[g]) * a.qk;
            attn_block<D, KSPLIT, CAUSAL, PV16, false, false, SEEDED>(
                odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, row, a.N, c, a.l448, h, r32, rsel, mref, lsum, O);
            kscale = knext;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
    for (; T < nblk; ++T) {
        const bool odd = T & 1;
        const bool more = T + 1 < nblk;
        const kvec knext = *reinterpret_cast<const kvec*>(ksc + KSPLIT * (more ? T + 1 : T));
        if (more) tiles.load(T + 1, odd ? lk0 : lk1, odd ? lv0 : lv1, wave);
        float c[KSPLIT];
#pragma unroll
        for (int g = 0; g < KSPLIT; ++g) c[g] = (sq * kscale[g]) * a.qk;
        // (without causality only the ragged last block is left here: one
        // body, whose registers then need no spilling at d = 128)
        if (CAUSAL && T < n_full)
            attn_block<D, KSPLIT, CAUSAL, PV16, false, false, SEEDED>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, row,
                                                       a.N, c, a.l448, h, r32, rsel, mref, lsum, O);
        else if (T <= wave_last)
            attn_block<D, KSPLIT, CAUSAL, PV16, true, false, SEEDED>(odd ? lk1 : lk0, odd ? lv1 : lv0, qf, T, row,
                                                      a.N, c, a.l448, h, r32, rsel, mref, lsum, O);
        kscale = knext;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: out = O * s_V / l.  O[ct][v] is channel 32ct + 8(v/4) + 4h + v%4.
    if (row >= a.N) return;
    const float* sv = a.v_scale + (long long)bg * D;
    const float inv_l = 1.0f / lsum;
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
}

// d = 64: 4-wave work-groups, two per CU (48 KB of LDS each), whose waves
// interleave on each SIMD.  d = 128: one 8-wave work-group per CU (96 KB of
// LDS), two waves per SIMD.  Either way a wave has half the register file,
// all of it architectural registers.
template <int D>
constexpr int attn_waves() {
#ifdef SAGE_ATTN_WAVES
    return SAGE_ATTN_WAVES;
#else
    return D == 64 ? 4 : 8;
#endif
}
template <int D>
constexpr int attn_waves_per_simd() {
#ifdef SAGE_ATTN_WPS
    return SAGE_ATTN_WPS;
#else
    return 2;
#endif
}

// Explicit instantiations: with the packed-FP32 feature switched off on the
// command line, this compiler otherwise leaves the host stubs of some of these
// kernels undefined.
#define SAGE_ATTN_INST(D, KSPLIT, CAUSAL, PV16, SEEDED)                                           \
    template __global__ void                                                                        \
    attn_fwd<D, KSPLIT, CAUSAL, PV16, SEEDED, attn_waves<D>(), attn_waves_per_simd<D>()>(AttnArgs);
#define SAGE_ATTN_INST_PV(D, KSPLIT, CAUSAL)                                                       \
    SAGE_ATTN_INST(D, KSPLIT, CAUSAL, false, true) SAGE_ATTN_INST(D, KSPLIT, CAUSAL, true, true)    \
    SAGE_ATTN_INST(D, KSPLIT, CAUSAL, false, false) SAGE_ATTN_INST(D, KSPLIT, CAUSAL, true, false)
SAGE_ATTN_INST_PV(64, 2, false)
SAGE_ATTN_INST_PV(64, 2, true)
SAGE_ATTN_INST_PV(64, 4, false)
SAGE_ATTN_INST_PV(64, 4, true)
SAGE_ATTN_INST_PV(128, 2, false)
SAGE_ATTN_INST_PV(128, 2, true)
SAGE_ATTN_INST_PV(128, 4, false)
SAGE_ATTN_INST_PV(128, 4, true)
#undef SAGE_ATTN_INST_PV
#undef SAGE_ATTN_INST

template <int D, int KSPLIT, bool CAUSAL, bool PV16, bool SEEDED>
static hipError_t launch_attn_t(AttnArgs a, hipStream_t st) {
    constexpr int WAVES = attn_waves<D>();
    constexpr int WPS = attn_waves_per_simd<D>();
    constexpr size_t lds = 2 * SAGE_BN * D + 2 * D * SAGE_BN * 2;
    a.nqt = a.Np / (32 * WAVES);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)attn_fwd<D, KSPLIT, CAUSAL, PV16, SEEDED, WAVES, WPS>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int total = a.B * a.Hq * a.nqt;
    hipLaunchKernelGGL((attn_fwd<D, KSPLIT, CAUSAL, PV16, SEEDED, WAVES, WPS>), dim3(total),
                       dim3(64 * WAVES), lds, st, a);
    return hipGetLastError();
}

template <int D, int KSPLIT, bool PV16, bool SEEDED>
static hipError_t launch_attn_p(AttnArgs a, int causal, hipStream_t st) {
    return causal ? launch_attn_t<D, KSPLIT, true, PV16, SEEDED>(a, st)
                  : launch_attn_t<D, KSPLIT, false, PV16, SEEDED>(a, st);
}

template <int D, int KSPLIT, bool PV16>
static hipError_t launch_attn_s(AttnArgs a, int causal, bool seeded, hipStream_t st) {
    return seeded ? launch_attn_p<D, KSPLIT, PV16, true>(a, causal, st)
                  : launch_attn_p<D, KSPLIT, PV16, false>(a, causal, st);
}

template <int D, int KSPLIT>
static hipError_t launch_attn_d(AttnArgs a, int causal, bool pv16, bool seeded, hipStream_t st) {
    return pv16 ? launch_attn_s<D, KSPLIT, true>(a, causal, seeded, st)
                : launch_attn_s<D, KSPLIT, false>(a, causal, seeded, st);
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
    a.q_shift = z->q_block == SAGE_BQ ? 7 : 0;  // SAGE_BQ = 128, SAGE_BQ_THREAD = 1
    a.qk = qk;
    a.l448 = l448;
    const bool fine_k = z->k_block == SAGE_BK_THREAD;  // 4 K scales per block, else 2
    const bool pv16 = z->pv_format == SAGE_PV_F16;
    const bool seeded = z->qk_bits == SAGE_QK_INT8;  // INT4 codes take the unseeded scores
    if (s.d == 64)
        return fine_k ? launch_attn_d<64, 4>(a, causal, pv16, seeded, st)
                      : launch_attn_d<64, 2>(a, causal, pv16, seeded, st);
    return fine_k ? launch_attn_d<128, 4>(a, causal, pv16, seeded, st)
                  : launch_attn_d<128, 2>(a, causal, pv16, seeded, st);
}

}  // namespace sage
