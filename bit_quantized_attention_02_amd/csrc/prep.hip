// The prep step of 8-bit quantized attention: K channel mean and smoothing,
// per-block INT8 of Q and smoothed K, per-channel E4M3 of V (SageAttention
// article: smoothing K and per-block INT8 Q/K; SageAttention2 summary: E4M3
// for V), or V's binary16 rounding for the binary16 P.V of the SageAttention
// article.  Memory-bound: every kernel streams 16-byte loads and does its
// reductions in registers, wavefront shuffles and LDS.
//
//   clear_words clears the per-kv-head arrival counters.
//   prep_qstats one launch for two independent jobs, so they overlap:
//               per (kv head, 512-row chunk): partial statistics (float64 K
//               channel sums, V channel absmax unless V goes to binary16),
//               and per (q head, 128-row block): Q absmax per scale group
//               (the block, or each row at the thread-level granularity),
//               scales and integer codes.  The head's last statistics work-group
//               to arrive (an atomic counter; nobody waits) reduces the
//               partials in a fixed chunk order (deterministic) into the K
//               mean and the V scales.
//   prep_pack   per (kv head, 64-row block) K - mean, absmax per scale group
//               (the block, or each 32-row half at the thread-level
//               granularity), scales, codes;
//               per (kv head, 128-key block) V E4M3 codes, stored as the
//               binary16 values they denote (or as code bytes for a KV cache,
//               or V's own binary16 rounding), transposed to the attention
//               kernels' channel-major, permuted-key layout.  Heads are
//               visited in the reverse order of the statistics so the second
//               read of K and V finds the most recent heads still in the
//               last-level cache.
// Q, K and V are read as contiguous [B, H, N, d] with constant offsets, or,
// when the caller passes other strides (a [B, N, H, d] tensor, a slice of a
// packed QKV tensor), through those strides: a template flag on the kernels,
// so the contiguous case keeps its offset arithmetic and registers.
#include "sage_internal.h"

namespace sage {

// Channels of V one prep_pack work-group transposes: all of them at d = 64;
// at d = 128 two work-groups take 64 each, so that the LDS tile (16 KB)
// leaves room for twice as many resident work-groups.
template <int D>
__host__ __device__ constexpr int pack_v_channels() {
    return D < 64 ? D : 64;
}

// The arrival counters of the statistics, one per kv head.
__host__ __device__ inline int sync_words(const Shape& s) { return s.B * s.Hkv; }

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ shared pieces
// Integer codes of 8 values with multiplier inv (RNE, clamped to +-qmax: 127
// for INT8, 7 for the INT4 values of the 4-bit variant), one byte each.
__device__ inline uint2 int8_codes(const float (&x)[8], float inv, float qmax) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float r = __builtin_rintf(x[i] * inv);
        r = fminf(fmaxf(r, -qmax), qmax);
        w[i >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * (i & 3));
    }
    return make_uint2(w[0], w[1]);
}

// Absolute maxima over groups of G rows (G a power of two dividing R, the
// work-group's rows).  On entry am[c] is this thread's absmax over the 8
// values of its chunk c, which lies in row (tid + c * kThreads) / CPR; on
// return it is the absmax over that row's group.  rmax and gmax are R floats
// of LDS each.
template <int CPR, int R, int NCH>
__device__ inline void group_absmax(float (&am)[NCH], int G, float* rmax, float* gmax) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int o = CPR / 2; o > 0; o >>= 1) am[c] = fmaxf(am[c], __shfl_xor(am[c], o));
    if (G == 1) return;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (tid % CPR == 0) rmax[(tid + c * kThreads) / CPR] = am[c];
    __syncthreads();
    const int span = G < 64 ? G : 64;  // rows reduced within one wavefront
    if (tid < R) {
        float m = rmax[tid];
        for (int o = 1; o < span; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        if ((tid & (span - 1)) == 0) gmax[tid / span] = m;
    }
    __syncthreads();
    const int per = G / span;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int g = (tid + c * kThreads) / CPR / G;
        float m = gmax[g * per];
        for (int j = 1; j < per; ++j) m = fmaxf(m, gmax[g * per + j]);
        am[c] = m;
    }
}

// The binary16 values of the E4M3 codes of x[i] * inv[i], i = 0..7, into the
// transposed V tile vt[D][SAGE_BN] at key position pos.
template <int D>
__device__ inline void v_codes_to_tile(const float (&x)[8], const float (&inv)[8], int col, int pos,
                                       uint16_t* vt) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        // |v * inv| <= 448 (1 + 2^-23); the clamp keeps the hardware
        // conversion (which gives NaN above 464) in range regardless.
        const float y0 = fminf(fmaxf(x[i] * inv[i], -448.0f), 448.0f);
        const float y1 = fminf(fmaxf(x[i + 1] * inv[i + 1], -448.0f), 448.0f);
        const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        // the binary16 value of each E4M3 code (exact).  The pair is read as
        // one 32-bit word: this compiler stores element [1] of the builtin's
        // vector result from the wrong half.
        const uint32_t h =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false));
        vt[(col + i) * SAGE_BN + pos] = (uint16_t)(h & 0xFFFFu);
        vt[(col + i + 1) * SAGE_BN + pos] = (uint16_t)(h >> 16);
    }
}

// The E4M3 code bytes of x[i] * inv[i], i = 0..7, into the transposed byte
// tile vt[D][SAGE_BN] at key position pos (a KV cache's V).
template <int D>
__device__ inline void v_codes_to_tile8(const float (&x)[8], const float (&inv)[8], int col, int pos,
                                        uint8_t* vt) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const float y0 = fminf(fmaxf(x[i] * inv[i], -448.0f), 448.0f);
        const float y1 = fminf(fmaxf(x[i + 1] * inv[i + 1], -448.0f), 448.0f);
        const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        vt[(col + i) * SAGE_BN + pos] = (uint8_t)(codes & 0xFF);
        vt[(col + i + 1) * SAGE_BN + pos] = (uint8_t)((codes >> 8) & 0xFF);
    }
}

// V's binary16 rounding (nearest even, clamped to +-65504 first so that
// out-of-range bf16 values saturate) of x[i], i = 0..7, into the transposed
// V tile.
template <int D>
__device__ inline void v_f16_to_tile(const float (&x)[8], int col, int pos, uint16_t* vt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const _Float16 h = (_Float16)fminf(fmaxf(x[i], -65504.0f), 65504.0f);
        vt[(col + i) * SAGE_BN + pos] = __builtin_bit_cast(uint16_t, h);
    }
}

// Copies a transposed V tile of VB-byte values from LDS to its place in the
// V operand (streaming stores: the tile is not read again by this step).
template <int D, int VB>
__device__ inline void store_v_tile(const void* vt, void* dst, int tid) {
    constexpr int OUT_CH = D * SAGE_BN * VB / 16 / kThreads;
#pragma unroll
    for (int c = 0; c < OUT_CH; ++c) {
        const int e = tid + c * kThreads;
        __builtin_nontemporal_store(*(reinterpret_cast<const v4u*>(vt) + e), reinterpret_cast<v4u*>(dst) + e);
    }
}

// ------------------------------------------------------------ Q
// Work-group qb codes 128 rows of a q head; one scale per bq rows (128 or 1).
// rmax and gmax are 128 floats of LDS each.
template <typename In, int D, bool STR>
__device__ inline void q_rows(const uint16_t* __restrict__ q, const Shape& s, int bq, float qmax,
                              int8_t* __restrict__ q_i8, float* __restrict__ q_scale, int qb,
                              float* rmax, float* gmax) {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    constexpr int R = 128;      // rows per work-group
    constexpr int NCH = R * CPR / kThreads;  // chunks per thread
    const int tid = threadIdx.x;
    const int nwg = s.Np / R;
    // rows [t*R, t*R+R) of head bh; rows >= N are zero padding
    const int bh = qb / nwg, t = qb % nwg;
    // (STR: Q read through its strides; otherwise contiguous, with constant offsets)
    const long long src_head = STR ? Shape::head_start(s.qs, bh, s.Hq) : (long long)bh * s.N * D;
    const long long qn = STR ? s.qs.n : D;
    const long long dst_head = (long long)bh * s.Np * D;
    // all of this thread's loads first (rows past N read row N-1 and are
    // zeroed), so they are in flight together
    uint4 u[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = tid + c * kThreads;
        const int row = min(t * R + e / CPR, s.N - 1), col = (e % CPR) * 8;
        u[c] = *reinterpret_cast<const uint4*>(q + src_head + (long long)row * qn + col);
    }
    // The values are unpacked twice (for the absmax, then for the codes)
    // rather than kept as floats across the group maximum: at d = 128 that
    // halves the registers, and the occupancy doubles.
    float am[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = tid + c * kThreads;
        const int row = t * R + e / CPR;
        float x[8];
        unpack8<In>(u[c], x);
        am[c] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am[c] = fmaxf(am[c], fabsf(x[i]));
        if (row >= s.N) am[c] = 0.0f;
    }
    group_absmax<CPR, R, NCH>(am, bq, rmax, gmax);
    const long long sbase = (long long)bh * (s.Np / bq);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = tid + c * kThreads;
        const int row = t * R + e / CPR, col = (e % CPR) * 8;
        const float a = am[c];
        if (e % CPR == 0 && row % bq == 0) q_scale[sbase + row / bq] = a / qmax;
        const float inv = a > 0.0f ? qmax / a : 0.0f;
        float x[8];
        unpack8<In>(u[c], x);
        if (row >= s.N) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.0f;
        }
        *reinterpret_cast<uint2*>(q_i8 + dst_head + (long long)row * D + col) = int8_codes(x, inv, qmax);
    }
}

// ------------------------------------------------------------ K and V
// Work-group wg sums one 512-row chunk of a kv head; the head's last chunk to
// arrive forms its K mean and V scales.
template <int D>
struct StatsSmem {
    static constexpr int RPI = kThreads / (D / 8);
    double ssum[RPI][D];
    float smax[RPI][D];
    int last;
};

template <typename In, int D, bool STR>
__device__ inline void kv_stats(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                const Shape& s, double* __restrict__ k_part,
                                float* __restrict__ v_part, int* __restrict__ cnt,
                                float* __restrict__ k_mean, float* __restrict__ v_scale,
                                float* __restrict__ v_inv, int pv16, int wg, StatsSmem<D>& sm) {
    constexpr int CPR = D / 8;
    constexpr int RPI = StatsSmem<D>::RPI;
    auto& ssum = sm.ssum;
    auto& smax = sm.smax;
    int& s_last = sm.last;
    const int tid = threadIdx.x;
    const int nchunk = s.part_chunks();
    const int bg = wg / nchunk, chunk = wg % nchunk;
    const int cg = tid % CPR, rr = tid / CPR;
    // contiguous inputs: one offset serves K and V; otherwise each its own
    const long long head = (long long)bg * s.N * D;
    const long long khead = STR ? Shape::head_start(s.ks, bg, s.Hkv) + cg * 8 : 0;
    const long long vhead = STR ? Shape::head_start(s.vs, bg, s.Hkv) + cg * 8 : 0;
    auto kv_load = [&](long long row, uint4& kk, uint4* vv) {
        if constexpr (STR) {
            kk = *reinterpret_cast<const uint4*>(k + khead + row * s.ks.n);
            if (vv) *vv = *reinterpret_cast<const uint4*>(v + vhead + row * s.vs.n);
        } else {
            const long long off = head + row * D + cg * 8;
            kk = *reinterpret_cast<const uint4*>(k + off);
            if (vv) *vv = *reinterpret_cast<const uint4*>(v + off);
        }
    };
    const int r0 = chunk * kStatRows;
    const int r1 = min(s.N, r0 + kStatRows);
    double sum[8];
    float mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sum[i] = 0.0;
        mx[i] = 0.0f;
    }
    // four rows per step, their loads issued together (the float64 sums of
    // 16-bit inputs are exact, so the order does not matter)
    constexpr int U = 4;
    int r = r0 + rr;
    for (; r + (U - 1) * RPI < r1; r += U * RPI) {
        uint4 uk[U], uv[U];
#pragma unroll
        for (int j = 0; j < U; ++j) kv_load(r + j * RPI, uk[j], pv16 ? nullptr : &uv[j]);
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float fk[8];
            unpack8<In>(uk[j], fk);
#pragma unroll
            for (int i = 0; i < 8; ++i) sum[i] += (double)fk[i];
            if (!pv16) {  // binary16 V needs no channel scale
                float fv[8];
                unpack8<In>(uv[j], fv);
#pragma unroll
                for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(fv[i]));
            }
        }
    }
    for (; r < r1; r += RPI) {
        uint4 uk1, uv1;
        kv_load(r, uk1, pv16 ? nullptr : &uv1);
        float fk[8];
        unpack8<In>(uk1, fk);
#pragma unroll
        for (int i = 0; i < 8; ++i) sum[i] += (double)fk[i];
        if (!pv16) {
            float fv[8];
            unpack8<In>(uv1, fv);
#pragma unroll
            for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(fv[i]));
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ssum[rr][cg * 8 + i] = sum[i];
        smax[rr][cg * 8 + i] = mx[i];
    }
    __syncthreads();
    if (tid < D) {
        double t = 0.0;
        float m = 0.0f;
        for (int r = 0; r < RPI; ++r) {
            t += ssum[r][tid];
            m = fmaxf(m, smax[r][tid]);
        }
        const long long o = ((long long)bg * nchunk + chunk) * D + tid;
        __hip_atomic_store(k_part + o, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(v_part + o, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Arrival.  The partials are written and read by device-scope atomic
    // accesses (coherent across the chip's L2 caches); waiting for the stores
    // to complete before the barrier and the arrival orders them, with no
    // cache writeback or invalidation.  Only the last work-group of the head
    // goes on; nobody waits.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(cnt + bg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 nchunk - 1;
    __syncthreads();
    if (!s_last) return;  // (uniform over the work-group)
    // The reduction over the head's chunks: LPC lanes per channel, each
    // loading every LPC-th chunk's partials with its loads in flight
    // together, then a fixed-order combination of the lanes through LDS.
    // (The float64 sums of 16-bit inputs are exact here, as above, so the
    // grouping does not change the result.)
    constexpr int LPC = kThreads / D;
    static_assert(LPC <= StatsSmem<D>::RPI, "the lanes' sums fit the stats buffers");
    {
        const int ch = tid % D, lane = tid / D;
        double t = 0.0;
        float m = 0.0f;
        constexpr int U = 8;
        const long long base = (long long)bg * nchunk * D + ch;
        int c = lane;
        for (; c + (U - 1) * LPC < nchunk; c += U * LPC) {
            double pk[U];
            float pv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pk[u] = __hip_atomic_load(k_part + base + (long long)(c + u * LPC) * D, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                pv[u] = __hip_atomic_load(v_part + base + (long long)(c + u * LPC) * D, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                t += pk[u];
                m = fmaxf(m, pv[u]);
            }
        }
        for (; c < nchunk; c += LPC) {
            t += __hip_atomic_load(k_part + base + (long long)c * D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            m = fmaxf(m, __hip_atomic_load(v_part + base + (long long)c * D, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
        }
        ssum[lane][ch] = t;
        smax[lane][ch] = m;
    }
    __syncthreads();
    if (tid >= D) return;
    double t = 0.0;
    float m = 0.0f;
    for (int l = 0; l < LPC; ++l) {
        t += ssum[l][tid];
        m = fmaxf(m, smax[l][tid]);
    }
    const long long o = (long long)bg * D + tid;
    k_mean[o] = (float)(t / (double)s.N);
    v_scale[o] = pv16 ? 1.0f : m / 448.0f;
    v_inv[o] = pv16 ? 1.0f : (m > 0.0f ? 448.0f / m : 0.0f);
}

// The K/V statistics and the Q codes in one launch: they read disjoint inputs,
// so they overlap.  Work-groups [0, nstats) take the statistics (the longer
// ones, dispatched first), the rest the Q row blocks (nq of them, 0 for a KV
// cache).  The arrival counters are cleared by clear_words beforehand.
template <typename In, int D, bool STR>
__global__ __launch_bounds__(kThreads) void prep_qstats(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    Shape s, int bq, float qmax, int8_t* __restrict__ q_i8, float* __restrict__ q_scale,
    double* __restrict__ k_part, float* __restrict__ v_part, int* __restrict__ cnt,
    float* __restrict__ k_mean, float* __restrict__ v_scale, float* __restrict__ v_inv, int pv16) {
    __shared__ StatsSmem<D> stats_smem;
    __shared__ float rmax[128], gmax[128];
    const int nstats = s.B * s.Hkv * s.part_chunks();
    const int wg = blockIdx.x;
    if (wg < nstats)
        kv_stats<In, D, STR>(k, v, s, k_part, v_part, cnt, k_mean, v_scale, v_inv, pv16, wg, stats_smem);
    else
        q_rows<In, D, STR>(q, s, bq, qmax, q_i8, q_scale, wg - nstats, rmax, gmax);
}

template <typename In, int D, bool STR>
__global__ __launch_bounds__(kThreads) void prep_pack(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, Shape s, int bk, float qmax,
    const float* __restrict__ k_mean, const float* __restrict__ v_inv,
    int8_t* __restrict__ k_i8, float* __restrict__ k_scale, void* __restrict__ v_out, int v_store) {
    constexpr int CPR = D / 8;
    constexpr int VC = pack_v_channels<D>();  // channels per V work-group
    __shared__ float rmax[64], gmax[64];
    __shared__ __attribute__((aligned(16))) uint16_t vt[VC * SAGE_BN];
    const int tid = threadIdx.x;
    const int nkb = s.Np / 64, nvb = s.Np / SAGE_BN;
    const int per_head = nkb + nvb * (D / VC);
    // reverse head order relative to the statistics
    const int bg = s.B * s.Hkv - 1 - (int)(blockIdx.x / per_head);
    const int j = blockIdx.x % per_head;

    if (j < nkb) {
        // K rows [t*64, t*64+64): smoothed, one scale per bk rows (64 or 32)
        const int t = j;
        constexpr int R = 64;
        constexpr int NCH = R * CPR / kThreads;
        const long long src_head = STR ? Shape::head_start(s.ks, bg, s.Hkv) : (long long)bg * s.N * D;
        const long long kn = STR ? s.ks.n : D;
        const long long dst_head = (long long)bg * s.Np * D;
        uint4 u[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int e = tid + c * kThreads;
            const int row = min(t * R + e / CPR, s.N - 1), col = (e % CPR) * 8;
            u[c] = *reinterpret_cast<const uint4*>(k + src_head + (long long)row * kn + col);
        }
        // a thread's column is the same in every chunk (kThreads % CPR == 0)
        float mean[8];
        {
            const float4* mp = reinterpret_cast<const float4*>(k_mean + (long long)bg * D + (tid % CPR) * 8);
            const float4 m0 = mp[0], m1 = mp[1];
            mean[0] = m0.x, mean[1] = m0.y, mean[2] = m0.z, mean[3] = m0.w;
            mean[4] = m1.x, mean[5] = m1.y, mean[6] = m1.z, mean[7] = m1.w;
        }
        float x[NCH][8], am[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int e = tid + c * kThreads;
            const int row = t * R + e / CPR;
            if (row < s.N) {
                unpack8<In>(u[c], x[c]);
#pragma unroll
                for (int i = 0; i < 8; ++i) x[c][i] = x[c][i] - mean[i];
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[c][i] = 0.0f;
            }
            am[c] = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) am[c] = fmaxf(am[c], fabsf(x[c][i]));
        }
        group_absmax<CPR, R, NCH>(am, bk, rmax, gmax);
        const long long sbase = (long long)bg * (s.Np / bk);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int e = tid + c * kThreads;
            const int row = t * R + e / CPR, col = (e % CPR) * 8;
            const float a = am[c];
            if (e % CPR == 0 && row % bk == 0) k_scale[sbase + row / bk] = a / qmax;
            const float inv = a > 0.0f ? qmax / a : 0.0f;
            *reinterpret_cast<uint2*>(k_i8 + dst_head + (long long)row * D + col) = int8_codes(x[c], inv, qmax);
        }
        return;
    }

    // V block T, channels [c0, c0 + VC): 128 keys x VC channels, transposed
    // through LDS.
    const int T = (j - nkb) / (D / VC), c0 = (j - nkb) % (D / VC) * VC;
    constexpr int CPRV = VC / 8;  // 16-byte chunks of a key's slice
    constexpr int NCH = SAGE_BN * CPRV / kThreads;
    static_assert(kThreads % CPRV == 0, "a thread keeps its column in every chunk");
    float inv[8];
    if (v_store != kVF16) {
        const float4* ip = reinterpret_cast<const float4*>(v_inv + (long long)bg * D + c0 + (tid % CPRV) * 8);
        const float4 i0 = ip[0], i1 = ip[1];
        inv[0] = i0.x, inv[1] = i0.y, inv[2] = i0.z, inv[3] = i0.w;
        inv[4] = i1.x, inv[5] = i1.y, inv[6] = i1.z, inv[7] = i1.w;
    }
    const long long src_head = STR ? Shape::head_start(s.vs, bg, s.Hkv) : (long long)bg * s.N * D;
    const long long vn = STR ? s.vs.n : D;
    uint4 u[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = tid + c * kThreads;
        const int row = min(T * SAGE_BN + e / CPRV, s.N - 1), col = c0 + (e % CPRV) * 8;
        u[c] = *reinterpret_cast<const uint4*>(v + src_head + (long long)row * vn + col);
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = tid + c * kThreads;
        const int key = e / CPRV, col = (e % CPRV) * 8;  // col: within the slice
        const int row = T * SAGE_BN + key;
        float x[8];
        unpack8<In>(u[c], x);
        if (row >= s.N) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.0f;
        }
        if (v_store == kVF16)
            v_f16_to_tile<VC>(x, col, v_key_position(key), vt);
        else if (v_store == kVE4M3Byte)
            v_codes_to_tile8<VC>(x, inv, col, v_key_position(key),
                                reinterpret_cast<uint8_t*>(vt));
        else
            v_codes_to_tile<VC>(x, inv, col, v_key_position(key), vt);
    }
    __syncthreads();
    // the slice's channels are a contiguous part of the block's [D][128] tile
    const long long tile = ((long long)bg * nvb + T) * (long long)(D * SAGE_BN) + (long long)c0 * SAGE_BN;
    if (v_store == kVE4M3Byte)
        store_v_tile<VC, 1>(vt, static_cast<uint8_t*>(v_out) + tile, tid);
    else
        store_v_tile<VC, 2>(vt, static_cast<uint16_t*>(v_out) + tile, tid);
}

// Clears the arrival counters of prep_qstats (one per kv head), before it.
__global__ __launch_bounds__(kThreads) void clear_words(int* __restrict__ w, int n) {
    for (int i = threadIdx.x; i < n; i += kThreads) w[i] = 0;
}

// ------------------------------------------------------------ launchers
// Counter clearing, then the statistics with the Q codes of nq row blocks
// (none for a KV cache), then the K and V codes.
template <typename In, int D, bool STR>
static hipError_t launch_prep_s(const void* q, const void* k, const void* v, const Shape& s,
                                int nq, int bq, float qmax, int8_t* q_i8, float* q_scale,
                                const KVViews& z, hipStream_t st) {
    hipLaunchKernelGGL(clear_words, dim3(1), dim3(kThreads), 0, st, z.sync, sync_words(s));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nstats = s.B * s.Hkv * s.part_chunks();
    const int pv16 = z.v_store == kVF16;
    hipLaunchKernelGGL((prep_qstats<In, D, STR>), dim3(nstats + nq), dim3(kThreads), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s, bq, qmax, q_i8,
                       q_scale, z.k_part, z.v_part, z.sync, z.k_mean, z.v_scale, z.v_inv, pv16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per_head = s.Np / 64 + s.Np / SAGE_BN * (D / pack_v_channels<D>());
    hipLaunchKernelGGL((prep_pack<In, D, STR>), dim3(s.B * s.Hkv * per_head), dim3(kThreads), 0, st,
                       (const uint16_t*)k, (const uint16_t*)v, s, z.k_block, z.qmax, z.k_mean, z.v_inv,
                       z.k_i8, z.k_scale, z.v, z.v_store);
    return hipGetLastError();
}

static bool is_contiguous(const InStrides& st, int H, int N, int d) {
    const InStrides c = contiguous_strides(H, N, d);
    return st.b == c.b && st.h == c.h && st.n == c.n;
}

// The kernels with constant offsets when every input is contiguous, else the
// ones that read through the strides.
template <typename In, int D>
static hipError_t launch_prep_all(const void* q, const void* k, const void* v, const Shape& s,
                                  int nq, int bq, float qmax, int8_t* q_i8, float* q_scale,
                                  const KVViews& z, hipStream_t st) {
    const bool contiguous = (nq == 0 || is_contiguous(s.qs, s.Hq, s.N, s.d)) &&
                            is_contiguous(s.ks, s.Hkv, s.N, s.d) && is_contiguous(s.vs, s.Hkv, s.N, s.d);
    return contiguous ? launch_prep_s<In, D, false>(q, k, v, s, nq, bq, qmax, q_i8, q_scale, z, st)
                      : launch_prep_s<In, D, true>(q, k, v, s, nq, bq, qmax, q_i8, q_scale, z, st);
}

template <typename In, int D>
static hipError_t launch_prep_t(const void* q, const void* k, const void* v, const Shape& s,
                                const sage_qkv_quant* z, hipStream_t st) {
    const float qmax = z->qk_bits == SAGE_QK_INT4 ? 7.0f : 127.0f;
    const KVViews kv = {z->k_i8,   z->k_scale, z->k_mean, z->v16,     z->v_scale,
                        z->v_inv,  z->k_part,  z->v_part, z->sync,    z->k_block,
                        z->pv_format == SAGE_PV_F16 ? kVF16 : kVE4M3Half, qmax};
    return launch_prep_all<In, D>(q, k, v, s, s.B * s.Hq * (s.Np / 128), (int)z->q_block, qmax,
                                  z->q_i8, z->q_scale, kv, st);
}

hipError_t launch_prep(const void* q, const void* k, const void* v, int dtype, const Shape& s,
                       const sage_qkv_quant* z, hipStream_t st) {
    if (dtype == SAGE_F16)
        return s.d == 64 ? launch_prep_t<_Float16, 64>(q, k, v, s, z, st)
                         : launch_prep_t<_Float16, 128>(q, k, v, s, z, st);
    return s.d == 64 ? launch_prep_t<Bf16Tag, 64>(q, k, v, s, z, st)
                     : launch_prep_t<Bf16Tag, 128>(q, k, v, s, z, st);
}

hipError_t launch_prep_kv(const void* k, const void* v, int dtype, const Shape& s, const KVViews& z,
                          hipStream_t st) {
    if (dtype == SAGE_F16)
        return s.d == 64 ? launch_prep_all<_Float16, 64>(nullptr, k, v, s, 0, 1, z.qmax, nullptr,
                                                         nullptr, z, st)
                         : launch_prep_all<_Float16, 128>(nullptr, k, v, s, 0, 1, z.qmax, nullptr,
                                                          nullptr, z, st);
    return s.d == 64 ? launch_prep_all<Bf16Tag, 64>(nullptr, k, v, s, 0, 1, z.qmax, nullptr, nullptr, z, st)
                     : launch_prep_all<Bf16Tag, 128>(nullptr, k, v, s, 0, 1, z.qmax, nullptr, nullptr,
                                                     z, st);
}

int prep_sync_words(const Shape& s) { return sync_words(s); }

}  // namespace sage
