// Fused 8-bit attention forward for CDNA4 (gfx950).
//
// One work-group = 4 waves = SAGE_BQ (128) query rows of one (batch, q head);
// each wave owns 32 rows as two 16-row groups.  The loop runs over blocks of
// SAGE_BN (128) keys:
//   1. the next block's INT8 K tile [128 x d] and FP8 V tile [d x 128] are
//      copied global -> LDS with global_load_lds (double-buffered, 16-byte
//      chunks XOR-swizzled so the fragment reads are bank-conflict free);
//   2. S^T = K Q^T on v_mfma_i32_16x16x64_i8 (INT8 x INT8 -> INT32, exact).
//      With keys on the M side, every lane ends up holding 32 scores of ONE
//      query row, so row maxima are in-lane plus two permlane swaps;
//   3. online softmax in FP32: block maximum m (on the INT32 scores, scaled
//      per K-scale half), P8 = e4m3(2^(s*c + log2(448) - m)) -- the block's
//      largest element codes to exactly 448 (SageAttention2's E4M3 P with a
//      per-block scale);
//   4. O^T += w * (V^T P^T) on v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales):
//      level 1 is one matrix-core product over the block's 128 keys, level 2
//      the FP32 register update O = alpha*O + w*acc (two-level accumulation;
//      the FP8 matrix core's internal sum is not full FP32, so blocks are not
//      chained through its accumulator).  The row sum of P comes out of the
//      same matrix core (an all-ones A operand), so the quantized weights are
//      normalised exactly.
// The P fragment a lane feeds to the P.V product is exactly the 32 scores it
// computed (keys 16*tau + 4*g + v for lane group g), so no data moves between
// lanes; V is stored by the prep kernel in that key order.
#include "sage_internal.h"

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct AttnArgs {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint8_t* v_fp8;
    const float* v_scale;
    float* out;
    int B, Hq, Hkv, N, Np, G, nqt;
    float qk;    // f32(sm_scale * log2 e)
    float l448;  // f32(log2 448)
};

// XOR swizzle of the 16-byte chunks of one K-tile row (d bytes long).
template <int D>
__device__ inline int kswz(int row) {
    return D == 64 ? ((row >> 1) & 3) : (row & 7);
}

__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)p;
}

// Copy key block T of this kv head (K: 128 rows x D, V: D rows x 128) into LDS.
template <int D>
__device__ inline void load_block(const uint8_t* kg, const uint8_t* vg, uint8_t* lk, uint8_t* lv,
                                  int wave, int lane) {
    constexpr int CPR = D / 16;     // 16-byte chunks per K row
    constexpr int ROUNDS = D / 32;  // (128*D/16) / 256 chunks per thread, same for V
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int p = r * kThreads + wave * 64 + lane;
        const int row = p / CPR, qs = p % CPR;
        const int q = qs ^ kswz<D>(row);
        __builtin_amdgcn_global_load_lds((const void*)(kg + row * D + q * 16),
                                         (__attribute__((address_space(3))) void*)(lk + (r * kThreads + wave * 64) * 16),
                                         16, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int p = r * kThreads + wave * 64 + lane;
        const int c = p >> 3, qs = p & 7;
        const int q = qs ^ (c & 7);
        __builtin_amdgcn_global_load_lds((const void*)(vg + c * SAGE_BN + q * 16),
                                         (__attribute__((address_space(3))) void*)(lv + (r * kThreads + wave * 64) * 16),
                                         16, 0, 0);
    }
}

__device__ inline int max_across_row(int x) {
    // the 4 lanes that hold one query row are l, l^16, l^32, l^48
    auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = max((int)a[0], (int)a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return max((int)b[0], (int)b[1]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd(AttnArgs a) {
    constexpr int KK = D / 64;   // 64-byte K chunks of a Q.K^T product
    constexpr int CT = D / 16;   // 16-channel tiles of the output
    __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][SAGE_BN * D];
    __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][D * SAGE_BN];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g16 = lane >> 4, r16 = lane & 15;

    // Work-group -> tile.  Consecutive work-groups are dispatched round-robin
    // over the 8 XCDs; give each XCD a contiguous range of tiles (same heads,
    // so K/V stay in that XCD's L2).
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
    const int q0 = qt * SAGE_BQ;

    const int nkb64 = a.Np / SAGE_BK;
    const int nblk = CAUSAL ? qt + 1 : a.Np / SAGE_BN;
    const int nfull = CAUSAL ? qt : (a.N % SAGE_BN == 0 ? nblk : nblk - 1);

    const int8_t* kbase = a.k_i8 + (long long)bg * a.Np * D;
    const uint8_t* vbase = a.v_fp8 + (long long)bg * a.Np * D;
    const float* ksc = a.k_scale + (long long)bg * nkb64;

    // Q fragments (B operand of the Q.K^T product): query row r16 of group qg,
    // bytes [64*kk + 16*g16, +16).
    v4i qf[2][KK];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int row = q0 + 32 * wave + 16 * qg + r16;
        const int8_t* qp = a.q_i8 + ((long long)bh * a.Np + row) * D + 16 * g16;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[qg][kk] = *reinterpret_cast<const v4i*>(qp + 64 * kk);
    }
    const float sq = a.q_scale[(long long)bh * a.nqt + qt];

    v4f O[2][CT];
    float m_run[2], l_run[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        m_run[qg] = -INFINITY;
        l_run[qg] = 0.0f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) O[qg][ct] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0

    load_block<D>((const uint8_t*)kbase, vbase, lds_k[0], lds_v[0], wave, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int T = 0; T < nblk; ++T) {
        const int buf = T & 1;
        if (T + 1 < nblk)
            load_block<D>((const uint8_t*)kbase + (long long)(T + 1) * SAGE_BN * D,
                          vbase + (long long)(T + 1) * SAGE_BN * D, lds_k[buf ^ 1],
                          lds_v[buf ^ 1], wave, lane);
        const uint8_t* lk = lds_k[buf];
        const uint8_t* lv = lds_v[buf];

        // ---- S^T = K Q^T (INT32)
        v4i S[2][8];
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
            const int row = 16 * tau + r16;
            v4i kf[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kf[kk] = *reinterpret_cast<const v4i*>(lk + row * D + (((4 * kk + g16) ^ kswz<D>(row)) << 4));
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
                v4i acc = {0, 0, 0, 0};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[kk], qf[qg][kk], acc, 0, 0, 0);
                S[qg][tau] = acc;
            }
        }

        const float sk0 = ksc[2 * T], sk1 = ksc[2 * T + 1];
        const float c0 = (sq * sk0) * a.qk, c1 = (sq * sk1) * a.qk;
        const bool masked = T >= nfull;

        v8i P[2];
        float alpha[2], wgt[2];
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const int row = q0 + 32 * wave + 16 * qg + r16;
            if (masked) {
#pragma unroll
                for (int tau = 0; tau < 8; ++tau)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int key = T * SAGE_BN + 16 * tau + 4 * g16 + v;
                        const bool off = (CAUSAL && key > row) || key >= a.N;
                        if (off) S[qg][tau][v] = INT32_MIN;
                    }
            }
            int M0 = INT32_MIN, M1 = INT32_MIN;
#pragma unroll
            for (int tau = 0; tau < 4; ++tau)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    M0 = max(M0, S[qg][tau][v]);
                    M1 = max(M1, S[qg][tau + 4][v]);
                }
            M0 = max_across_row(M0);
            M1 = max_across_row(M1);
            const float m0 = M0 == INT32_MIN ? -INFINITY : (float)M0 * c0;
            const float m1 = M1 == INT32_MIN ? -INFINITY : (float)M1 * c1;
            const float mt = fmaxf(m0, m1);
            const float bias = a.l448 - mt;
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) {
                const float c = tau < 4 ? c0 : c1;
                float y[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    y[v] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)S[qg][tau][v], c, bias));
                    if (masked && S[qg][tau][v] == INT32_MIN) y[v] = 0.0f;
                }
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
                P[qg][tau] = w;
            }
            const float m_new = fmaxf(m_run[qg], mt);
            alpha[qg] = m_run[qg] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[qg] - m_new);
            wgt[qg] = mt == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mt - m_new);
            m_run[qg] = m_new;
        }

        // ---- O^T = alpha O^T + w (V^T P^T), row sums from the same products
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int c = 16 * ct + r16;
            const uint8_t* vr = lv + c * SAGE_BN;
            const v4i lo = *reinterpret_cast<const v4i*>(vr + (((2 * g16) ^ (c & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(vr + (((2 * g16 + 1) ^ (c & 7)) << 4));
            const v8i vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
                const v4f z = {0.f, 0.f, 0.f, 0.f};
                const v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    vf, P[qg], z, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    O[qg][ct][v] = __builtin_fmaf(acc[v], wgt[qg], O[qg][ct][v] * alpha[qg]);
            }
        }
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const v4f z = {0.f, 0.f, 0.f, 0.f};
            const v4f rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P[qg], z, 0, 0, 0,
                                                                            127, 0, 127);
            l_run[qg] = __builtin_fmaf(rs[0], wgt[qg], l_run[qg] * alpha[qg]);
        }

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: out = O * s_V / l
    const float* sv = a.v_scale + (long long)bg * D;
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int row = q0 + 32 * wave + 16 * qg + r16;
        if (row >= a.N) continue;
        const float inv_l = 1.0f / l_run[qg];
        float* op = a.out + ((long long)bh * a.N + row) * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int ch = 16 * ct + 4 * g16;
            const float4 s4 = *reinterpret_cast<const float4*>(sv + ch);
            float4 o;
            o.x = O[qg][ct][0] * s4.x * inv_l;
            o.y = O[qg][ct][1] * s4.y * inv_l;
            o.z = O[qg][ct][2] * s4.z * inv_l;
            o.w = O[qg][ct][3] * s4.w * inv_l;
            *reinterpret_cast<float4*>(op + ch) = o;
        }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
    const int total = a.B * a.Hq * a.nqt;
    hipLaunchKernelGGL((attn_fwd<D, CAUSAL>), dim3(total), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn(const sage_qkv_quant* z, float* out, const Shape& s, int causal,
                       float qk, float l448, hipStream_t st) {
    AttnArgs a;
    a.q_i8 = z->q_i8;
    a.q_scale = z->q_scale;
    a.k_i8 = z->k_i8;
    a.k_scale = z->k_scale;
    a.v_fp8 = z->v_fp8;
    a.v_scale = z->v_scale;
    a.out = out;
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.Np = s.Np;
    a.G = s.Hq / s.Hkv;
    a.nqt = s.Np / SAGE_BQ;
    a.qk = qk;
    a.l448 = l448;
    if (s.d == 64) return causal ? launch_attn_t<64, true>(a, st) : launch_attn_t<64, false>(a, st);
    return causal ? launch_attn_t<128, true>(a, st) : launch_attn_t<128, false>(a, st);
}

}  // namespace sage
