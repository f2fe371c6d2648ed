/*
 * CPU oracle for the forward pass of 8-bit quantized attention (SageAttention
 * with the FP8 P.V of SageAttention2).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; it is written from
 * the method's description alone, as plain loops in a fixed order, in float64
 * except where a quantisation decision is defined on float32 values.
 *
 * Sources (SageAttention article, "对 K 进行平滑处理" / "对 Q, K 进行分块 INT8
 * 量化" paragraphs; SageAttention2 summary on the INT4-quantisation search page,
 * item (4) on P and V; the Berkeley news brief's technique checklist):
 *   - K is smoothed by subtracting its mean over tokens, per channel; softmax
 *     is unchanged because the subtracted term is constant along each row.
 *   - Q and K are quantised to INT8 per block of rows (the flash tile), QK^T
 *     is an INT8 product with INT32 accumulation.
 *   - P and V are quantised to FP8 E4M3; V per channel, P per block, and P.V
 *     is accumulated in two levels (within a block, then across blocks).
 *
 * Readings where the pages are silent (each is a parameter of the spec the
 * HIP path implements too):
 *   - INT8 is symmetric, range +-127, round-to-nearest-even of x*(127/absmax)
 *     evaluated in float32; an all-zero block gets scale 0 and codes 0.
 *   - The 4-bit Q, K of SageAttention2 (INT4; the Berkeley brief's comparison
 *     table) are the same with 7 in place of 127: codes in [-7, 7], scale
 *     absmax/7.  The codes are stored one per byte and multiplied like the
 *     INT8 codes.
 *   - E4M3 is OCP E4M3FN (bias 7, max 448, subnormal step 2^-9), RNE,
 *     saturating at +-448; V codes are e4m3(v * (448/absmax_c)) in float32.
 *   - The softmax runs in FP32 (the method's online softmax): the integer
 *     score acc (exact, |acc| < 2^24) is converted to float32 exactly and
 *     multiplied by the score factor c = f32(f32(s_q * s_k) * f32(sm_scale *
 *     log2 e)), one float32 rounding: s = f32(acc * c), in log2 units.
 *   - The P block is one query row by `bn` keys.  Its scale is the block
 *     maximum over 448 (the Berkeley brief's softmax-domain scaling): with mt
 *     the block's largest s (float32), P8 = e4m3(2^x) with x = f32(acc * c +
 *     f32(f32(log2 448) - mt)) (one fused multiply-add), so the largest
 *     element codes to 448, and the block enters the second accumulation
 *     level with weight 2^(mt - M), M the row maximum.  The row sum l is the
 *     same two-level sum over the quantised P, so the quantised weights are
 *     normalised exactly.  See oracle_attn_q.  The P8 decision is taken on
 *     this float32 x; only 2^x itself is evaluated in float64 here.  Codes
 *     whose 2^x lies within a relative `tau` of a rounding midpoint have two
 *     correct values (an FP32 exp2 may round either way); the oracle returns
 *     the interval spanned by both choices.
 *
 * The binary16 P.V mode (SageAttention article, paragraph on the P, V product:
 * P and V stay FP16 there, with an FP16 accumulator).  The matrix cores this
 * library targets accumulate binary16 products in FP32 only, so the mode keeps
 * P and V in IEEE binary16 and the two accumulation levels in FP32/float64:
 *   - V16 = f16(v), round to nearest even, saturating at +-65504; no V scale.
 *   - P16 = f16(2^x) with x as above but log2(448) replaced by 0, so the
 *     block's largest element is exactly 1 (P stays in (0, 1]).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- E4M3 codec */

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent 0 is
 * subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN; no infinities. */
double oracle_e4m3_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* Round-to-nearest-even to E4M3FN, saturating at +-448. */
uint8_t oracle_e4m3_encode(double x) {
    uint8_t s = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (isnan(x)) return (uint8_t)(s | 0x7F);
    if (a >= 448.0) return (uint8_t)(s | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; rint is round-half-even.  A
         * result of 8 is the smallest normal, whose code is also 8. */
        double r = rint(ldexp(a, 9));
        return (uint8_t)(s | (uint8_t)r);
    }
    int ex;
    frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;          /* a in [2^e, 2^(e+1)) */
    double r = rint(ldexp(a, 3 - e)); /* mantissa with 3 fraction bits, in [8,16] */
    if (r == 16.0) {
        r = 8.0;
        e += 1;
    }
    return (uint8_t)(s | (uint8_t)(((e + 7) << 3) | ((int)r - 8)));
}

void oracle_e4m3_encode_array(const double* x, long n, uint8_t* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_decode_array(const uint8_t* c, long n, double* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------ binary16 codec */

/* IEEE 754 binary16: sign, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 is subnormal (m * 2^-24); exponent 31 is infinity (m = 0) or NaN. */
double oracle_f16_decode(uint16_t code) {
    int s = code >> 15, e = (code >> 10) & 31, m = code & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* Round-to-nearest-even to binary16, saturating at +-65504 (no infinities
 * from finite inputs). */
uint16_t oracle_f16_encode(double x) {
    uint16_t s = signbit(x) ? 0x8000 : 0x0000;
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(s | 0x7E00);
    if (a >= 65504.0) return (uint16_t)(s | 0x7BFF);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-24; a result of 1024 is the
         * smallest normal, whose code is also 1024 */
        return (uint16_t)(s | (uint16_t)rint(ldexp(a, 24)));
    }
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                        /* a in [2^e, 2^(e+1)) */
    double r = rint(ldexp(a, 10 - e));     /* 10 fraction bits: r in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    return (uint16_t)(s | (uint16_t)(((e + 15) << 10) | ((int)r - 1024)));
}

void oracle_f16_encode_array(const double* x, long n, uint16_t* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_f16_encode(x[i]);
}

void oracle_f16_decode_array(const uint16_t* c, long n, double* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_f16_decode(c[i]);
}

/* ------------------------------------------------------------ quantisation */

/* Symmetric integer codes of one block of `count` float32 values, in
 * [-qmax, qmax] (qmax = 127 for INT8, 7 for INT4). */
static void quant_block_i8(const float* x, long count, int qmax, int8_t* out, float* scale) {
    const float qm = (float)qmax;
    float a = 0.0f;
    for (long i = 0; i < count; ++i) {
        float m = fabsf(x[i]);
        if (m > a) a = m;
    }
    if (a == 0.0f) {
        *scale = 0.0f;
        memset(out, 0, (size_t)count);
        return;
    }
    float inv = qm / a;
    *scale = a / qm;
    for (long i = 0; i < count; ++i) {
        float t = rintf(x[i] * inv);
        if (t > qm) t = qm;
        if (t < -qm) t = -qm;
        out[i] = (int8_t)t;
    }
}

/*
 * The prep step: K mean and smoothing, per-block INT8 of Q and smoothed K,
 * per-channel E4M3 of V.  Inputs are float32 copies of the fp16/bf16 tensors
 * (the up-conversion is exact), layout [B, H, N, d].  The Q half and the K/V
 * half are independent (a KV cache is the K/V half over the cached tokens,
 * and a short query the Q half over its own rows).
 *
 * Outputs (all caller-allocated):
 *   q_i8 [B,Hq,N,d], q_scale [B,Hq,ceil(N/bq)]
 *   k_i8 [B,Hkv,N,d], k_scale [B,Hkv,ceil(N/bk)], k_mean [B,Hkv,d]
 *   v_fp8 [B,Hkv,N,d] (E4M3 codes), v_scale [B,Hkv,d]
 * smooth = 0 skips the K mean (ablation only; k_mean is then all zero).
 */
void oracle_quantize_q(const float* q, int B, int Hq, int N, int d, int bq, int qmax,
                       int8_t* q_i8, float* q_scale) {
    const long nd = (long)N * d;
    const int nqb = (N + bq - 1) / bq;
    /* one scale per (b, h, block of bq rows) */
#pragma omp parallel for collapse(2) schedule(static)
    for (int bh = 0; bh < B * Hq; ++bh)
        for (int t = 0; t < nqb; ++t) {
            long r0 = (long)t * bq, r1 = r0 + bq < N ? r0 + bq : N;
            quant_block_i8(q + bh * nd + r0 * d, (r1 - r0) * d, qmax, q_i8 + bh * nd + r0 * d,
                           q_scale + (long)bh * nqb + t);
        }
}

void oracle_quantize_kv(const float* k, const float* v, int B, int Hkv, int N, int d, int bk,
                        int qmax, int smooth, int8_t* k_i8, float* k_scale, float* k_mean,
                        uint8_t* v_fp8, float* v_scale) {
    const long nd = (long)N * d;
    const int nkb = (N + bk - 1) / bk;

#pragma omp parallel for schedule(static)
    for (int bg = 0; bg < B * Hkv; ++bg) {
        const float* kh = k + bg * nd;
        const float* vh = v + bg * nd;
        float* mean = k_mean + (long)bg * d;
        /* K mean over all N tokens, per channel: float64 sum, one rounding. */
        for (int c = 0; c < d; ++c) {
            double s = 0.0;
            for (long n = 0; n < N; ++n) s += (double)kh[n * d + c];
            mean[c] = smooth ? (float)(s / (double)N) : 0.0f;
        }
        /* Smoothed K in float32, then per-block INT8 over bk rows. */
        float* ks = (float*)malloc(sizeof(float) * (size_t)nd);
        for (long n = 0; n < N; ++n)
            for (int c = 0; c < d; ++c) ks[n * d + c] = kh[n * d + c] - mean[c];
        for (int t = 0; t < nkb; ++t) {
            long r0 = (long)t * bk, r1 = r0 + bk < N ? r0 + bk : N;
            quant_block_i8(ks + r0 * d, (r1 - r0) * d, qmax, k_i8 + bg * nd + r0 * d,
                           k_scale + (long)bg * nkb + t);
        }
        free(ks);
        /* V per channel: absmax over tokens, E4M3 of v * (448/absmax). */
        for (int c = 0; c < d; ++c) {
            float a = 0.0f;
            for (long n = 0; n < N; ++n) {
                float m = fabsf(vh[n * d + c]);
                if (m > a) a = m;
            }
            float* sv = v_scale + (long)bg * d + c;
            if (a == 0.0f) {
                *sv = 0.0f;
                for (long n = 0; n < N; ++n) v_fp8[bg * nd + n * d + c] = 0;
                continue;
            }
            float inv = 448.0f / a;
            *sv = a / 448.0f;
            for (long n = 0; n < N; ++n) {
                float t = vh[n * d + c] * inv;
                v_fp8[bg * nd + n * d + c] = oracle_e4m3_encode((double)t);
            }
        }
    }
}

void oracle_quantize(const float* q, const float* k, const float* v,
                     int B, int Hq, int Hkv, int N, int d, int bq, int bk, int qmax, int smooth,
                     int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                     float* k_mean, uint8_t* v_fp8, float* v_scale) {
    oracle_quantize_q(q, B, Hq, N, d, bq, qmax, q_i8, q_scale);
    oracle_quantize_kv(k, v, B, Hkv, N, d, bk, qmax, smooth, k_i8, k_scale, k_mean, v_fp8, v_scale);
}

/* ------------------------------------------------- quantised attention */

/*
 * Quantised attention of Nq query rows per head against Nk keys, for a list of
 * query rows (flattened (b*Hq + h)*Nq + i; rows == NULL means every row).
 * Query row i sits at key position i + Nk - Nq (the last Nq positions of the
 * sequence: Nq = Nk is self-attention, Nq < Nk a short query against a longer
 * KV cache).  For each row, with g = h / (Hq/Hkv) and the allowed keys
 * j <= i + Nk - Nq (causal) or all j < Nk:
 *
 *   acc_j = sum_c q_i8[i,c] * k_i8[j,c]                       (exact integer)
 *   c_j   = f32( f32(sq * f32(sm_scale*log2 e)) * sk[j/bk] )   (float32)
 *   s_j   = f32(acc_j * c_j)                                   (float32, log2 units)
 *   blocks t of bn keys; m_t = max of s_j over the block's allowed keys
 *   x_j   = fmaf(acc_j, c_j, f32(f32(log2 448) - m_t))
 *   y_j   = 2^x_j (float64);  P8_j = e4m3(y_j)   (the block maximum codes to 448)
 *   level 1: A_t[c] = sum_{j in t} P8_j * V8[j,c];  R_t = sum_{j in t} P8_j
 *   level 2: with M = max_t m_t and w_t = 2^(m_t - M) (float64),
 *            O[c] = sum_t w_t A_t[c],  l = sum_t w_t R_t
 *   out[c] = O[c] * sv[c] / l
 *
 * pv_f16 = 1 selects the binary16 P.V mode: v_codes holds binary16 codes of V
 * (uint16), v_scale may be NULL (sv = 1), f32(log2 448) above is replaced by 0
 * and P16_j = f16(y_j) replaces P8_j; the rest is unchanged.
 *
 * out_lo/out_hi (optional) bound the output over every choice of the P8 codes
 * whose y lies within relative distance tau of a rounding midpoint: changing
 * code j by delta moves out[c] by w delta (V8[j,c] sv[c] - out[c]) / (l + w
 * delta); the bounds add these moves' negative and positive parts, widened by
 * their relative interaction (sum |w delta| / l).  flagged (optional)
 * receives the number of such codes per row.
 */
void oracle_attn_q(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                   const float* k_scale, const void* v_codes, const float* v_scale, int pv_f16,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, int bq, int bk, int bn,
                   int causal, float sm_scale, double tau, const int64_t* rows, long nrows,
                   double* out, double* out_lo, double* out_hi, int64_t* flagged) {
    const long qnd = (long)Nq * d, nd = (long)Nk * d;
    const int N = Nk; /* keys */
    const int G = Hq / Hkv;
    const int nqb = (Nq + bq - 1) / bq, nkb = (N + bk - 1) / bk;
    const float qk = (float)((double)sm_scale * 1.4426950408889634); /* log2(e) */
    /* the P block scale: the block maximum maps to 448 (E4M3) or to 1 (binary16) */
    const float l448 = pv_f16 ? 0.0f : (float)log2(448.0);
    /* decoded value of every code of the P.V format, and its largest finite
     * positive code */
    const int ncode = pv_f16 ? 65536 : 256;
    const int top = pv_f16 ? 0x7BFF : 0x7E;
    double* dec = (double*)malloc(sizeof(double) * (size_t)ncode);
    for (int i = 0; i < ncode; ++i)
        dec[i] = pv_f16 ? oracle_f16_decode((uint16_t)i) : oracle_e4m3_decode((uint8_t)i);
    const uint8_t* v8 = (const uint8_t*)v_codes;
    const uint16_t* v16 = (const uint16_t*)v_codes;
    if (rows == NULL) nrows = (long)B * Hq * Nq;

#pragma omp parallel
    {
        int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
        float* cj = (float*)malloc(sizeof(float) * (size_t)N);
        float* aj = (float*)malloc(sizeof(float) * (size_t)N);
        float* mblk = (float*)malloc(sizeof(float) * (size_t)(N / bn + 2));
        double* A = (double*)malloc(sizeof(double) * (size_t)d);
        double* O = (double*)malloc(sizeof(double) * (size_t)d);
        int32_t* fj = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);   /* flagged keys */
        double* fwd = (double*)malloc(sizeof(double) * (size_t)N);     /* their w * delta */
#pragma omp for schedule(dynamic, 1)
        for (long ri = 0; ri < nrows; ++ri) {
            long row = rows ? (long)rows[ri] : ri;
            long bh = row / Nq;
            int i = (int)(row % Nq);
            int b = (int)(bh / Hq), h = (int)(bh % Hq);
            int g = h / G;
            const int8_t* qrow = q_i8 + bh * qnd + (long)i * d;
            const int8_t* kh = k_i8 + ((long)b * Hkv + g) * nd;
            const long vhead = ((long)b * Hkv + g) * nd;
            const float* svh = v_scale ? v_scale + ((long)b * Hkv + g) * d : NULL;
            const float sq = q_scale[bh * nqb + i / bq];
            const float* skh = k_scale + ((long)b * Hkv + g) * nkb;
            /* causal needs Nq <= Nk, so that every row keeps key 0 */
            int jmax = causal ? i + (Nk - Nq) : N - 1;
            int nt = jmax / bn + 1;

            /* scores */
            for (int j = 0; j <= jmax; ++j) {
                int32_t s = 0;
                const int8_t* kr = kh + (long)j * d;
                for (int c = 0; c < d; ++c) s += (int32_t)qrow[c] * (int32_t)kr[c];
                acc[j] = s;
                float sqq = sq * qk;
                cj[j] = sqq * skh[j / bk];
                aj[j] = (float)s; /* exact: |acc| < 2^24 */
            }
            /* per-block maximum score: the P scale of the block */
            float M = -INFINITY;
            for (int t = 0; t < nt; ++t) {
                int j0 = t * bn, j1 = j0 + bn - 1 < jmax ? j0 + bn - 1 : jmax;
                float mt = -INFINITY;
                for (int j = j0; j <= j1; ++j) {
                    float s = aj[j] * cj[j];
                    if (s > mt) mt = s;
                }
                mblk[t] = mt;
                if (mt > M) M = mt;
            }
            /* P quantisation and the two-level accumulation */
            double l = 0.0;
            int64_t nflag = 0;
            for (int c = 0; c < d; ++c) O[c] = 0.0;
            for (int t = 0; t < nt; ++t) {
                int j0 = t * bn, j1 = j0 + bn - 1 < jmax ? j0 + bn - 1 : jmax;
                float bias = l448 - mblk[t];
                double w = exp2((double)mblk[t] - (double)M);
                double R = 0.0;
                for (int c = 0; c < d; ++c) A[c] = 0.0;
                for (int j = j0; j <= j1; ++j) {
                    float x = fmaf(aj[j], cj[j], bias);
                    double y = exp2((double)x);
                    int code = pv_f16 ? (int)oracle_f16_encode(y) : (int)oracle_e4m3_encode(y);
                    double p = dec[code];
                    R += p;
                    const long vr = vhead + (long)j * d;
                    if (pv_f16)
                        for (int c = 0; c < d; ++c) A[c] += p * dec[v16[vr + c]];
                    else
                        for (int c = 0; c < d; ++c) A[c] += p * dec[v8[vr + c]];
                    if (out_lo || flagged) {
                        /* the other code is also correct when y sits within
                         * tau of the midpoint to a neighbouring code */
                        double alt = p;
                        if (code < top) {
                            double up = dec[code + 1], mid = 0.5 * (p + up);
                            if (fabs(y - mid) <= tau * mid) alt = up;
                        }
                        if (code > 0 && alt == p) {
                            double dn = dec[code - 1], mid = 0.5 * (p + dn);
                            if (fabs(y - mid) <= tau * mid) alt = dn;
                        }
                        if (alt != p) {
                            fj[nflag] = j;
                            fwd[nflag] = w * (alt - p);
                            ++nflag;
                        }
                    }
                }
                for (int c = 0; c < d; ++c) O[c] += w * A[c];
                l += w * R;
            }
            for (int c = 0; c < d; ++c) out[ri * d + c] = O[c] * (svh ? (double)svh[c] : 1.0) / l;
            if (out_lo) {
                double inter = 0.0;
                for (int64_t e = 0; e < nflag; ++e) inter += fabs(fwd[e]) / l;
                for (int c = 0; c < d; ++c) {
                    double o = out[ri * d + c], neg = 0.0, pos = 0.0;
                    for (int64_t e = 0; e < nflag; ++e) {
                        const long vi = vhead + (long)fj[e] * d + c;
                        double vjc = (pv_f16 ? dec[v16[vi]] : dec[v8[vi]]) * (svh ? (double)svh[c] : 1.0);
                        double mv = fwd[e] * (vjc - o) / (l + fwd[e]);
                        if (mv < 0) neg += mv;
                        else pos += mv;
                    }
                    double slack = 2.0 * inter * (pos - neg);
                    out_lo[ri * d + c] = o + neg - slack;
                    out_hi[ri * d + c] = o + pos + slack;
                }
            }
            if (flagged) flagged[ri] = nflag;
        }
        free(acc);
        free(cj);
        free(aj);
        free(mblk);
        free(A);
        free(O);
        free(fj);
        free(fwd);
    }
    free(dec);
}

/* ------------------------------------------- full-precision attention */

/*
 * softmax(Q K^T * sm_scale) V in float64 for a list of rows (same row
 * indexing as oracle_attn_q: Nq query rows at the last Nq of Nk positions),
 * with the causal mask j <= i + Nk - Nq when asked.  Inputs are float64,
 * q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d].
 */
void oracle_attn_f64(const double* q, const double* k, const double* v, int B, int Hq,
                     int Hkv, int Nq, int Nk, int d, int causal, double sm_scale,
                     const int64_t* rows, long nrows, double* out) {
    const long qnd = (long)Nq * d, nd = (long)Nk * d;
    const int N = Nk;
    const int G = Hq / Hkv;
    if (rows == NULL) nrows = (long)B * Hq * Nq;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (long ri = 0; ri < nrows; ++ri) {
            long row = rows ? (long)rows[ri] : ri;
            long bh = row / Nq;
            int i = (int)(row % Nq);
            int b = (int)(bh / Hq), h = (int)(bh % Hq);
            int g = h / G;
            const double* qr = q + bh * qnd + (long)i * d;
            const double* kh = k + ((long)b * Hkv + g) * nd;
            const double* vh = v + ((long)b * Hkv + g) * nd;
            int jmax = causal ? i + (Nk - Nq) : N - 1;
            double m = -INFINITY;
            for (int j = 0; j <= jmax; ++j) {
                double t = 0.0;
                for (int c = 0; c < d; ++c) t += qr[c] * kh[(long)j * d + c];
                s[j] = t * sm_scale;
                if (s[j] > m) m = s[j];
            }
            double l = 0.0;
            double* o = out + ri * d;
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            for (int j = 0; j <= jmax; ++j) {
                double p = exp(s[j] - m);
                l += p;
                for (int c = 0; c < d; ++c) o[c] += p * vh[(long)j * d + c];
            }
            for (int c = 0; c < d; ++c) o[c] /= l;
        }
        free(s);
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
