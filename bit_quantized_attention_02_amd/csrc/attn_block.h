// One 128-key block of 8-bit quantized attention for one wave of 32 query
// rows on CDNA4 (gfx950): the device code shared by the prefill kernel
// (attn_fwd.hip) and the short-query kernel over a quantized KV cache
// (attn_decode.hip).
//
// Per block of SAGE_BN (128) keys:
//   1. the next block's INT8 K tile [128 x d] and V tile [d x 128] (binary16
//      copies of the E4M3 codes) are copied global -> LDS by buffer loads that
//      write LDS directly, double-buffered, with 16-byte chunks XOR-swizzled
//      so the fragment reads are free of bank conflicts;
//   2. S^T = K Q^T on v_mfma_i32_32x32x32_i8 (INT8 x INT8 -> INT32, exact).
//      With keys on the M side every lane holds 64 scores of ONE query row,
//      and the other 64 sit in the lane 32 apart: a row maximum is in-lane
//      work plus one permlane32 swap;
//   3. online softmax in FP32.  Each score enters float32 exactly (see
//      ScoreConv): at d = 64 by one conversion per score; at d = 128, where
//      the matrix pipe has room and the vector ALU does not, on the matrix
//      pipe: the accumulator is seeded with a float32 bit pattern, so a tile
//      read as float32 is an exact affine image of the integer scores, and
//      one v_mfma_f32_16x16x1_4b_f32 per tile removes the offset from all 16
//      values of a lane at once, exactly.
//      Block maximum m = f32(max acc * c) per K-scale group (on the integer
//      patterns, which order like the scores), and
//      P8 = e4m3(2^fmaf(acc, c, f32(log2(448) - m))), so the block's largest
//      element codes to exactly 448 (the E4M3 P with a per-block scale);
//   4. level 1: the block's P8.V8 product on v_mfma_f32_32x32x16_f16 -- the
//      E4M3 values are exact in binary16 and that matrix core sums the exact
//      products in FP32 (gfx950's FP8 matrix core truncates its internal sum to
//      about 2^-11 of the largest product, too coarse for rows dominated by a
//      single key); level 2: the FP32 register update O += w * acc with
//      w = 2^(m - reference max).  The row sum of P comes out of the 16x16
//      binary16 matrix core (a 0/1 operand, see row_sum_selector), so the
//      quantized weights are normalised exactly.  P is converted 16 keys at a
//      time and each piece goes to the matrix core at once, so the
//      conversions of one piece run while the products of the previous one
//      are in flight.
// The binary16 P.V variant (the SageAttention article's own P.V, with FP32
// accumulation) differs only in step 3: P16 = f16(2^(acc*c - m)), one
// rounding instead of the E4M3 round trip, and V holds V's binary16 rounding
// with scale 1.
// The reference max is raised lazily, only when a block's maximum exceeds it
// by more than 8 (log2 units), so O is rescaled rarely.
// The P operand a lane feeds to P.V is exactly the scores it computed, so
// nothing moves between lanes; V is stored by the prep kernel in that order.
#pragma once

#include "sage_internal.h"

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr float kLazyRescale = 8.0f;

// How the INT32 scores of a tile become float32, exactly, per head dimension.
// Every ScoreConv<D> yields F = kF * acc for each integer score acc, with the
// factor applied to the score factor instead (c' = kF^-1 * c, exact: kF is a
// power of two up to sign), so F * c' = acc * c in every product.
//  d = 64: no seed; F = f32(acc) by v_cvt_f32_i32 (kF = 1).  A masked score
//          (INT32_MIN) becomes -2^31, which no real score reaches.
//  d = 128: the accumulator is seeded with the pattern 0xCBC80000, the
//          float32 -1.5625 * 2^24; with |acc| < 2^21 (127^2 * 128 < 2^21) the
//          pattern + acc stays in that binade and reads as the float32
//          -(1.5625 * 2^24) - 2 acc.  v_mfma_f32_16x16x1_4b_f32 with A = B =
//          5120 (5120^2 = 1.5625 * 2^24, one register for both operands)
//          adds the constant back to all 16 values of a lane: F = -2 acc,
//          exact, the two terms sharing their binade (kF = -2).  A masked
//          score (INT32_MIN, read as -0.0) becomes +1.5625 * 2^24.
//  The integer patterns order like the scores in both cases, so the row
//  maximum is taken on them.
// Score factors passed to the block body: one per K-scale group (KSPLIT of
// 2 or 4 per block), c = f32(f32(s_q * f32(sm_scale * log2 e)) * s_k), or,
// with one K scale per key (KSPLIT == SAGE_BN), the row's part f32(s_q *
// f32(sm_scale * log2 e)) alone, the keys' scales coming from LDS.
template <int KSPLIT>
constexpr int score_factors() {
    return KSPLIT == SAGE_BN ? 1 : KSPLIT;
}

template <int D> struct ScoreConv;
template <> struct ScoreConv<64> {
    static constexpr int kSeedBits = 0;
    static constexpr float kInvF = 1.0f;           // c' = kInvF * c
    static constexpr float kMasked = -2147483648.0f;
    static __device__ __forceinline__ v16f to_f32(const v16i& s) { return __builtin_convertvector(s, v16f); }
    static __device__ __forceinline__ float max_to_f32(int m) { return (float)m; }
};
template <> struct ScoreConv<128> {
    static constexpr int kSeedBits = (int)0xCBC80000u;
    static constexpr float kSeed = 26214400.0f;    // 5120^2 = -(the seed's value)
    static constexpr float kInvF = -0.5f;
    static constexpr float kMasked = 26214400.0f;
    static __device__ __forceinline__ v16f to_f32(const v16i& s) {
        return __builtin_amdgcn_mfma_f32_16x16x1f32(5120.0f, 5120.0f, __builtin_bit_cast(v16f, s), 0, 0, 0);
    }
    static __device__ __forceinline__ float max_to_f32(int m) { return __builtin_bit_cast(float, m) + kSeed; }
};

// XOR swizzle of the 16-byte chunks of one K-tile row (d bytes long): the 16
// lanes of one LDS read phase (16 consecutive rows, same chunk) land on 16
// different 16-byte bank groups.
template <int D>
__host__ __device__ constexpr int kswz(int row) {
    return D == 64 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}
// and of one V-tile row (a channel: 128 binary16 = 16 chunks, or 128 E4M3
// bytes = 8 chunks).  With bytes, the 32 lanes of one 8-byte read phase
// (32 channels, same chunk) cover 32 of the 64 banks twice: a 2-way conflict,
// the least a 16-byte swizzle allows for 8-byte reads.
__host__ __device__ constexpr int vswz(int ch) { return ch & 15; }
__host__ __device__ constexpr int vswz8(int ch) { return (ch >> 1) & 7; }
template <int VB>
__host__ __device__ constexpr int vswz_b(int ch) {
    return VB == 2 ? vswz(ch) : vswz8(ch);
}

// Smallest number of load steps after which a lane's swizzled offset repeats,
// shifted by whole steps: each step moves `step` rows down the tile, and the
// swizzle is periodic in the row.
template <int VB, bool IS_K, int D>
constexpr int swizzle_period(int step, int steps) {
    for (int p = 1; p < steps; p *= 2) {
        bool same = true;
        for (int row = 0; row < 256; ++row)
            if ((IS_K ? kswz<D>(row + p * step) : vswz_b<VB>(row + p * step)) !=
                (IS_K ? kswz<D>(row) : vswz_b<VB>(row)))
                same = false;
        if (same) return p;
    }
    return steps;
}

// Copies key blocks (K: 128 rows x D bytes, V: D rows x 128 values of VB
// bytes, binary16 or E4M3) of one kv head into LDS with buffer loads that
// write LDS directly.  Load step r copies LDS chunks [r NT, (r+1) NT); a
// lane's global offset in step r is its offset in step r % P (P the swizzle
// period) plus whole steps, which go in the scalar offset with the block's
// base, so a block costs no vector ALU work and only P offset registers per
// tile.
template <int D, int WAVES, int VB = 2>
struct TileLoader {
    static constexpr int NT = 64 * WAVES;
    static constexpr int KR = SAGE_BN * D / 16 / NT;       // 16-byte chunks per lane, K
    static constexpr int VR = D * SAGE_BN * VB / 16 / NT;  // and V
    static constexpr int VCH = SAGE_BN * VB / 16;          // 16-byte chunks per V row
    static_assert(KR * NT * 16 == SAGE_BN * D && VR * NT * 16 == D * SAGE_BN * VB,
                  "tile must split evenly over the work-group");
    static constexpr int KP = swizzle_period<VB, true, D>(NT * 16 / D, KR);
    static constexpr int VP = swizzle_period<VB, false, D>(NT / VCH, VR);
    static_assert(KR % KP == 0 && VR % VP == 0, "load steps must cover whole periods");
    __amdgpu_buffer_rsrc_t krs, vrs;
    uint32_t koff[KP], voff[VP];

    __device__ TileLoader(const uint8_t* kg, const void* vg, int head_rows, int wave, int lane) {
        krs = __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, head_rows * D, 0x00020000);
        vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, head_rows * D * VB, 0x00020000);
#pragma unroll
        for (int r = 0; r < KP; ++r) {
            // LDS chunk p of the K tile holds chunk p ^ swizzle of its row
            const int p = r * NT + wave * 64 + lane;
            const int row = p / (D / 16), qs = p % (D / 16);
            koff[r] = row * D + ((qs ^ kswz<D>(row)) << 4);
        }
#pragma unroll
        for (int r = 0; r < VP; ++r) {
            const int p = r * NT + wave * 64 + lane;
            const int c = p / VCH, qs = p % VCH;
            voff[r] = c * (SAGE_BN * VB) + ((qs ^ vswz_b<VB>(c)) << 4);
        }
    }

    // KR instructions
    __device__ inline void load_k(int T, uint8_t* lk, int wave) const {
#pragma unroll
        for (int r = 0; r < KR; ++r)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                krs, (__attribute__((address_space(3))) void*)(lk + (r * NT + wave * 64) * 16), 16,
                koff[r % KP], T * SAGE_BN * D + (r / KP) * KP * NT * 16, 0, 0);
    }
    // VR instructions
    __device__ inline void load_v(int T, void* lv, int wave) const {
#pragma unroll
        for (int r = 0; r < VR; ++r)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrs, (__attribute__((address_space(3))) void*)((uint8_t*)lv + (r * NT + wave * 64) * 16),
                16, voff[r % VP], T * SAGE_BN * D * VB + (r / VP) * VP * NT * 16, 0, 0);
    }
    // K then V
    __device__ inline void load(int T, uint8_t* lk, void* lv, int wave) const {
        load_k(T, lk, wave);
        load_v(T, lv, wave);
    }
};

// A operand of v_mfma_f32_16x16x32_f16 that turns a P piece into row sums.
// Read as that shape's B operand, a P piece puts lane l's 8 values in column
// l%16, reduction rows 8(l/16)..8(l/16)+7.  Lane l holds keys of query l%32,
// so column n mixes query n (lane quarters 0 and 2) with query n+16 (quarters
// 1 and 3).  Output rows 4G..4G+3 land in lane quarter G, whose own query is
// n + 16(G%2); A[m][k] = 1 exactly when (k/8)%2 == (m/4)%2 sums the two
// quarters of that query, so each lane receives its own row's sum over the
// piece's 16 keys (in all four output registers).  Lane l supplies
// A[l%16][8(l/16)..+8]: ones when (l/16)%2 == (l%16/4)%2, else zeros.
__device__ inline v8h row_sum_selector(int lane) {
    const _Float16 x = (((lane >> 4) ^ (lane >> 2)) & 1) ? (_Float16)0.0f : (_Float16)1.0f;
    const v8h r = {x, x, x, x, x, x, x, x};
    return r;
}

// An 8-byte LDS read as one vector load.  (Read as a uint2 structure it is
// split into two scalar loads that carry no type-based alias information, and
// the compiler then makes them wait for every copy into LDS still in flight,
// such as the next block's K tile.)
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2u lds_read8(const uint8_t* p) {
    return *reinterpret_cast<const v2u*>(p);
}

// Maximum over the two lanes (l, l^32) that hold one query row.
__device__ inline int max_across_halves(int x) {
    auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((int)a[0], (int)a[1]);
}

// S^T = K Q^T of one key block for one wave (32 query rows), INT32, on
// v_mfma_i32_32x32x32_i8.  Tile t, element v: key 32t + 8(v/4) + 4h + v%4.
// The accumulator starts from ScoreConv<D>::kSeedBits.
template <int D>
__device__ __forceinline__ void block_scores(const uint8_t* __restrict__ lk, const v4i (&qf)[D / 32],
                                             int h, int r32, v16i (&S)[4]) {
    constexpr int KS = D / 32;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int kr = 32 * t + r32;
        v16i acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = ScoreConv<D>::kSeedBits;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v4i kf = *reinterpret_cast<const v4i*>(lk + kr * D + (((2 * ks + h) ^ kswz<D>(kr)) << 4));
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[ks], acc, 0, 0, 0);
        }
        S[t] = acc;
    }
}

// The rest of one key block for one wave, from its scores S: masking, online
// softmax, P and both levels of P.V.  MASKED: some keys of the block are
// excluded (causal diagonal, or keys >= N).  PV16: P is rounded to binary16
// directly (l448 is then 0) instead of through E4M3.  V8: the V tile holds
// E4M3 code bytes (a KV cache), converted to binary16 -- exactly -- as each
// fragment is read.
// KSPLIT: K scales per block of SAGE_BN keys (2: one per 64 keys; 4: one per
// 32-key tile; SAGE_BN: one per key).  For 2 or 4, c[g] is the score factor
// f32(f32(s_q * f32(sm_scale * log2 e)) * s_k) of scale group g; tile t
// belongs to group t / (4 / KSPLIT).  For SAGE_BN, c[0] is the row's part
// f32(s_q * f32(sm_scale * log2 e)) and the block's 128 key scales are at
// lks in LDS; each key's factor f32(c[0] * s_k) is formed where it is needed.
template <int D, int KSPLIT, bool CAUSAL, bool PV16, bool MASKED, bool V8 = false>
__device__ __forceinline__ void block_softmax_pv(v16i (&S)[4], const void* __restrict__ lv, int T,
                                                 int row, int N, const float (&c)[score_factors<KSPLIT>()],
                                                 float l448, int h, int r32, const v8h& rsel, float& mref,
                                                 float& lsum, v16f (&O)[D / 32],
                                                 const float* __restrict__ lks = nullptr) {
    constexpr int CT = D / 32;
    constexpr bool PER_KEY = KSPLIT == SAGE_BN;
    constexpr int NG = PER_KEY ? 1 : KSPLIT;  // scale groups held in registers
    constexpr int TPG = 4 / NG;               // tiles per scale group
    typedef ScoreConv<D> SC;
    float cf[NG];  // the factors of the converted scores F (F * cf = acc * c)
    if constexpr (!PER_KEY) {
#pragma unroll
        for (int g = 0; g < KSPLIT; ++g) cf[g] = c[g] * SC::kInvF;
    }
    // per key: the factor of key 32t + 8i + 4h + j (element 4i + j of tile
    // t), f32(row part * s_k) times the power of two kInvF (exact), one
    // product per key
    const float rowf = PER_KEY ? c[0] * SC::kInvF : 0.0f;
    auto key_factor = [&](int t, int i, int j) -> float {
        const v4f ks = *reinterpret_cast<const v4f*>(lks + 32 * t + 8 * i + 4 * h);
        return rowf * ks[j];
    };

    // ---- block maxima, one per K-scale group
    if (MASKED) {
        const int rel = row - T * SAGE_BN;  // this lane's row, relative to the block
        const int lim = N - T * SAGE_BN;    // keys at or past this are padding
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int kr = 32 * t + 8 * (v >> 2) + 4 * h + (v & 3);
                if ((CAUSAL && kr > rel) || kr >= lim) S[t][v] = INT32_MIN;
            }
    }
    float mt = -INFINITY;
    v16f F[4];
    if constexpr (PER_KEY) {
        // the scores as float32 first, then the largest f32(acc * c_key)
#pragma unroll
        for (int t = 0; t < 4; ++t) F[t] = SC::to_f32(S[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float f = F[t][4 * i + j];
                    const float sc = f * key_factor(t, i, j);
                    if (!MASKED || f != SC::kMasked) mt = fmaxf(mt, sc);
                }
        // (the other half of the row's keys sit in the lane 32 apart)
        const auto both = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, mt), __builtin_bit_cast(int, mt),
                                                           false, false);
        mt = fmaxf(__builtin_bit_cast(float, (int)both[0]), __builtin_bit_cast(float, (int)both[1]));
    } else {
#pragma unroll
        for (int g = 0; g < KSPLIT; ++g) {
            int M = S[g * TPG][0];
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt)
#pragma unroll
                for (int v = (tt == 0 ? 1 : 0); v < 16; ++v) M = max(M, S[g * TPG + tt][v]);
            M = max_across_halves(M);
            // f32(acc_max * c), one rounding: the largest f32(acc * c) of the
            // group, since c >= 0
            float m = SC::max_to_f32(M) * cf[g];
            if (MASKED && M == INT32_MIN) m = -INFINITY;
            mt = fmaxf(mt, m);
        }
        // the scores as float32 (see ScoreConv)
#pragma unroll
        for (int t = 0; t < 4; ++t) F[t] = SC::to_f32(S[t]);
    }

    // ---- lazy update of the reference maximum
    {
        const float nr = mt > mref + kLazyRescale ? mt : mref;
        const bool up = nr > mref;
        if (__any(up)) {
            const float alpha = up ? __builtin_amdgcn_exp2f(mref - nr) : 1.0f;
            lsum *= alpha;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int v = 0; v < 16; ++v) O[ct][v] *= alpha;
        }
        mref = nr;
    }
    const float w = mt == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mt - mref);

    // ---- P in pieces of 16 keys (8 per lane), each straight into level 1.
    // At d = 128 the channel tiles go in two passes of two, so that one pass's
    // accumulators, the P pieces and O fit in the architectural registers.
    constexpr int CG = CT < 2 ? CT : 2;
    const float bias = l448 - mt;
    v8h P[8];
    v4f rs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int pass = 0; pass < CT / CG; ++pass) {
        v16f acc[CG];
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (pass == 0) {
                const int t = s >> 1, base = 8 * (s & 1);
                const float ct = PER_KEY ? 0.0f : cf[t / TPG];
                v4i quad;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    float y[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int v = base + 4 * g + i;
                        const float cv = PER_KEY ? key_factor(t, v >> 2, v & 3) : ct;
                        y[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(F[t][v], cv, bias));
                        if (MASKED && F[t][v] == SC::kMasked) y[i] = 0.0f;
                    }
                    if (PV16) {
                        // round to nearest even, two values per conversion
                        const v2f lo = {y[0], y[1]}, hi = {y[2], y[3]};
                        quad[2 * g] = __builtin_bit_cast(int, __builtin_convertvector(lo, v2h));
                        quad[2 * g + 1] = __builtin_bit_cast(int, __builtin_convertvector(hi, v2h));
                    } else {
                        // the first conversion writes the low half; the high
                        // half of its destination is then written by the
                        // second, so the register's old contents never matter
                        // (the builtin would zero it first)
                        int code;
                        asm("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(code) : "v"(y[0]), "v"(y[1]));
                        code = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], code, true);
                        quad[2 * g] = __builtin_bit_cast(
                            int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, false));
                        quad[2 * g + 1] = __builtin_bit_cast(
                            int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, true));
                    }
                }
                P[s] = __builtin_bit_cast(v8h, quad);
                rs = __builtin_amdgcn_mfma_f32_16x16x32_f16(rsel, P[s], rs, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < CG; ++j) {
                const int ch = 32 * (pass * CG + j) + r32;
                v8h vf;
                if (V8) {
                    // keys 16s + 8h .. +8 of the channel: 8 code bytes
                    const v2u raw = lds_read8(
                        (const uint8_t*)lv + ch * SAGE_BN + ((s ^ vswz8(ch)) << 4) + 8 * h);
                    const v4i w = {
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.x, 1.0f, false)),
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.x, 1.0f, true)),
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.y, 1.0f, false)),
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.y, 1.0f, true))};
                    vf = __builtin_bit_cast(v8h, w);
                } else {
                    vf = *reinterpret_cast<const v8h*>((const uint16_t*)lv + ch * SAGE_BN +
                                                       (((2 * s + h) ^ vswz(ch)) << 3));
                }
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, P[s], acc[j], 0, 0, 0);
            }
        }
        // ---- level 2 in FP32 registers
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                O[pass * CG + j][v] = __builtin_fmaf(acc[j][v], w, O[pass * CG + j][v]);
    }
    lsum = __builtin_fmaf(rs[0], w, lsum);
}

// One whole key block for one wave: block_scores, then block_softmax_pv.
template <int D, int KSPLIT, bool CAUSAL, bool PV16, bool MASKED, bool V8 = false>
__device__ __forceinline__ void attn_block(const uint8_t* __restrict__ lk,
                                           const void* __restrict__ lv,
                                           const v4i (&qf)[D / 32], int T, int row, int N,
                                           const float (&c)[score_factors<KSPLIT>()], float l448, int h,
                                           int r32, const v8h& rsel, float& mref, float& lsum,
                                           v16f (&O)[D / 32], const float* __restrict__ lks = nullptr) {
    v16i S[4];
    block_scores<D>(lk, qf, h, r32, S);
    block_softmax_pv<D, KSPLIT, CAUSAL, PV16, MASKED, V8>(S, lv, T, row, N, c, l448, h, r32, rsel,
                                                          mref, lsum, O, lks);
}

}  // namespace sage
