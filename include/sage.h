/*
 * sage.h -- C ABI of the MI355X (gfx950) 8-bit quantized attention library.
 *
 * The method (SageAttention, with the FP8 P.V of SageAttention2):
 *   - K is smoothed by subtracting its per-channel mean over all tokens
 *     (SageAttention article, paragraph on smoothing K: softmax(QK^T) equals
 *     softmax(Q(K - mean K)^T) because the subtracted term is constant along
 *     each row);
 *   - Q and smoothed K are quantized to INT8 per block of rows at the flash
 *     tile granularity and Q.K^T runs as INT8 x INT8 with INT32 accumulation
 *     (same article, paragraph on per-block INT8 quantization of Q and K);
 *   - the softmax is computed online in FP32;
 *   - P and V are quantized to FP8 E4M3, V per channel and P per block, and
 *     P.V is accumulated in two levels (SageAttention2 summary on the
 *     INT4-quantization search page, item (4) on P and V; the Berkeley news
 *     brief's checklist: outlier smoothing, block-wise scales, two-level
 *     accumulation, softmax-domain scaling).
 *
 * Spec details the pages leave open (the CPU oracle under oracle/ follows the
 * same ones):
 *   - INT8: symmetric, +-127, code = rne(x * f32(127/absmax)) in float32; an
 *     all-zero block has scale 0.  Three granularities: per block (the default:
 *     one Q scale per SAGE_BQ query rows, one K scale per SAGE_BK keys, the
 *     flash tile of the SageAttention article) and thread-level (one Q scale
 *     per query row -- each lane of the attention kernel owns one row -- and
 *     one K scale per 32-key matrix-core tile; the Berkeley brief's checklist
 *     item on thread-level block quantization); and token granularity (one
 *     Q scale per query row and one K scale per key, the finest the scheme
 *     allows: the attention kernel forms each key's score factor where it
 *     needs it, at a cost in vector work, for the rows whose large |Q| the
 *     coarser K groups quantize too coarsely).  sage_qkv_quant.q_block and
 *     .k_block select it.
 *   - FP8: OCP E4M3FN (max 448), round to nearest even.  V: one scale per
 *     channel, code = e4m3(v * f32(448/absmax_c)).
 *   - Softmax in FP32: each integer score acc (exact) becomes float32 exactly
 *     and, in log2 units, f32(acc * c) with c = f32(f32(s_q *
 *     f32(sm_scale*log2 e)) * s_k) (the row's part formed first, so that a
 *     per-key factor costs one product per key).
 *   - P: one block is one query row by SAGE_BN keys; with m the block's
 *     largest f32(acc * c), the block's codes are
 *     e4m3(2^fmaf(acc, c, f32(f32(log2(448)) - m))), so the largest element
 *     codes to 448.  Level 1 is the block's P8.V8 product, exact products
 *     summed in FP32 by the matrix core; level 2 adds it, weighted by
 *     2^(m - reference max), into FP32 registers.  The row sum is the same
 *     weighted sum of the quantized P.
 *   - P.V format (sage_qkv_quant.pv_format).  SAGE_PV_E4M3 is the above.
 *     SAGE_PV_F16 is the SageAttention article's own P.V (paragraph on the P, V
 *     product: P and V stay FP16): V is its binary16 rounding (round to nearest
 *     even, saturating at +-65504) with no scale, and P is
 *     f16(2^fmaf(acc, c, -m)), so the block's largest element is exactly 1.
 *     The article accumulates in FP16; the binary16 matrix cores here
 *     accumulate in FP32 only, so both levels stay FP32.
 *   - Q, K code width (sage_qkv_quant.qk_bits).  SAGE_QK_INT4 gives the
 *     numerics of SageAttention2's 4-bit Q, K (the SageAttention2 summary;
 *     the Berkeley brief's comparison table) as an accuracy option, not a
 *     faster path: the INT8 scheme with 7 in place of 127 (codes in [-7, 7],
 *     scale absmax/7), stored one code per byte and multiplied on the INT8
 *     matrix core (gfx950 has no INT4 one), at INT8 speed.  Decode caches are
 *     INT8 only.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Tensors are contiguous
 *     [B, H, N, d] with d innermost (the *_strided entry points also read
 *     Q, K, V in other layouts); Q has Hq heads, K and V have Hkv heads,
 *     query head h reads kv head h / (Hq/Hkv).
 *   - Q, K, V and out must be 16-byte aligned; the workspace 256-byte aligned.
 *   - Supported: d in {64, 128}; N >= 1; B, Hq, Hkv >= 1; Hq % Hkv == 0;
 *     N <= SAGE_MAX_N.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; device-side faults surface at the
 *     caller's next synchronisation.
 *   - Argument errors are detected on the host before any HIP call and return
 *     a negative sage_status; nothing is enqueued then.  A failed launch
 *     returns SAGE_ERR_HIP.  No C++ exception crosses this interface.
 *   - Non-finite inputs give unspecified output.
 *   - Calls that share a workspace must not overlap (same stream, or ordered).
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_BQ 128       /* query rows per Q scale */
#define SAGE_BK 64        /* keys per K scale */
#define SAGE_BN 128       /* keys per P block (one step of the attention loop) */
#define SAGE_FP8_MAX 448  /* largest finite E4M3FN value */
#define SAGE_NPAD 256     /* sequence padding of the quantized operands */
#define SAGE_MAX_N (1 << 20)
#define SAGE_BQ_THREAD 1  /* query rows per Q scale, thread-level granularity */
#define SAGE_BK_THREAD 32 /* keys per K scale, thread-level granularity */
#define SAGE_BK_TOKEN 1   /* keys per K scale, token granularity (one scale per key) */
#define SAGE_PV_E4M3 0    /* P and V as FP8 E4M3 (the default) */
#define SAGE_PV_F16 1     /* P and V as binary16 */
#define SAGE_QK_INT8 8    /* Q, K codes: INT8 (the default) */
#define SAGE_QK_INT4 4    /* Q, K codes: INT4 values in [-7, 7], one per byte */

typedef enum {
    SAGE_OK = 0,
    SAGE_ERR_INVALID_ARG = -1, /* null or misaligned pointer, bad flag, bad size */
    SAGE_ERR_UNSUPPORTED = -2, /* d not in {64,128}, Hq % Hkv != 0, N too large, unknown
                                  granularity or P.V format */
    SAGE_ERR_WORKSPACE = -3,   /* workspace too small or misaligned */
    SAGE_ERR_HIP = -4          /* a HIP launch failed */
} sage_status;

typedef enum { SAGE_F16 = 0, SAGE_BF16 = 1 } sage_dtype;

typedef struct {
    int bq, bk, bn;  /* SAGE_BQ, SAGE_BK, SAGE_BN */
    int fp8_max;     /* 448: FP8 is OCP E4M3FN */
    int version;     /* library version, 100 * major + minor */
} sage_config;

/*
 * Device-side views of the quantized operands inside a workspace (filled by
 * sage_workspace_carve).  N_p = N rounded up to a multiple of SAGE_NPAD; rows
 * N..N_p-1 are zero padding.  bq = q_block, bk = k_block below.
 *   q_i8    int8 [B, Hq, N_p, d]            row-major, d innermost
 *   q_scale f32  [B, Hq, N_p / bq]
 *   k_i8    int8 [B, Hkv, N_p, d]           codes of K - k_mean
 *   k_scale f32  [B, Hkv, N_p / bk]          (room for bk = 1)
 *   k_mean  f32  [B, Hkv, d]
 *   v16     binary16 [B, Hkv, N_p / SAGE_BN, d, SAGE_BN]: the V operand of
 *           P.V.  With SAGE_PV_E4M3, the E4M3 codes of V, each stored as the
 *           binary16 number it denotes (exact: every E4M3 value is a binary16
 *           value), so the product runs on the binary16 matrix core with exact
 *           products; with SAGE_PV_F16, V's own binary16 rounding.  For each
 *           block of SAGE_BN keys and each channel, the block's values in the
 *           key order of sage_v_key_position()
 *   v_scale f32  [B, Hkv, d]                absmax / 448 per channel (1 with SAGE_PV_F16)
 *   v_inv   f32  [B, Hkv, d]                448 / absmax, 0 for a zero channel (1 with SAGE_PV_F16)
 *   k_part, v_part: per-chunk partial statistics used by sage_quantize.
 *   sync    int32 [B * Hkv]: per-kv-head arrival counters of the statistics
 *           kernel of sage_quantize, which clears them itself on every call.
 *   tail_part f32 [tail_rows, d + 2]: partial results of the attention call's
 *           last partial round.  When the non-causal tiles do not fill whole
 *           rounds of the work-groups the GPU runs at once, the leftover
 *           tiles are split along the keys and their shares merged; NULL (or
 *           too few tail_rows for a split) runs them whole.  Same results up
 *           to FP32 rounding.  Set by sage_workspace_carve (d = 64 only).
 */
typedef struct {
    int8_t* q_i8;
    float* q_scale;
    int8_t* k_i8;
    float* k_scale;
    float* k_mean;
    uint16_t* v16;
    float* v_scale;
    float* v_inv;
    double* k_part;
    float* v_part;
    int32_t* sync;
    int32_t q_block; /* query rows per Q scale: SAGE_BQ (set by sage_workspace_carve) or SAGE_BQ_THREAD */
    int32_t k_block; /* keys per K scale: SAGE_BK (set by sage_workspace_carve), SAGE_BK_THREAD or
                        SAGE_BK_TOKEN */
    int32_t pv_format; /* SAGE_PV_E4M3 (set by sage_workspace_carve) or SAGE_PV_F16; the
                          attention call must see the value the quantize call saw */
    int32_t qk_bits;   /* SAGE_QK_INT8 (set by sage_workspace_carve) or SAGE_QK_INT4; likewise */
    float* tail_part;   /* may be NULL */
    int64_t tail_rows;  /* rows of tail_part (0 with NULL) */
    int32_t B, Hq, Hkv, N, d; /* the shape the views were carved for (set by
                                 sage_workspace_carve); the quantize and attention
                                 calls return SAGE_ERR_INVALID_ARG for other sizes */
} sage_qkv_quant;

/* Method options of sage_attn_fwd_ex. */
typedef struct {
    int32_t q_block;   /* SAGE_BQ or SAGE_BQ_THREAD */
    int32_t k_block;   /* SAGE_BK, SAGE_BK_THREAD or SAGE_BK_TOKEN (paired with q_block as above) */
    int32_t pv_format; /* SAGE_PV_E4M3 or SAGE_PV_F16 */
    int32_t qk_bits;   /* SAGE_QK_INT8 or SAGE_QK_INT4 */
} sage_options;

/* Bytes of workspace sage_quantize/sage_attn_fwd need for this shape (0 when
 * the shape is invalid). */
size_t sage_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/* Split `workspace` (device memory, 256-byte aligned, ws_bytes long) into the
 * views above, with the per-block granularity (q_block = SAGE_BQ, k_block =
 * SAGE_BK) and E4M3 P.V; the caller may then switch the block sizes to
 * (SAGE_BQ_THREAD, SAGE_BK_THREAD) or (SAGE_BQ_THREAD, SAGE_BK_TOKEN) (the
 * workspace holds the scales of any of them) and pv_format to SAGE_PV_F16.  The quantize and attention calls
 * given the struct read these fields; any other values make them return
 * SAGE_ERR_UNSUPPORTED.  Host-only; no HIP call. */
int sage_workspace_carve(void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int N, int d,
                         sage_qkv_quant* out);

/*
 * The prep step (K mean, smoothing, per-block INT8 of Q and K, per-channel
 * FP8 of V, or V's binary16 rounding with SAGE_PV_F16) from fp16/bf16 Q, K, V
 * into the views of `dst` (carved for these sizes).  Memory-bound; runs as three kernels on
 * `stream`: clearing of the arrival counters; the K/V statistics (whose last
 * work-group per kv head forms the K mean and V scales) together with the Q
 * codes; the K/V codes.
 */
int sage_quantize(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                  int N, int d, const sage_qkv_quant* dst, void* stream);

/*
 * Attention on already-quantized operands: out = softmax(Q K^T sm_scale) V as
 * the method computes it, FP32 output [B, Hq, N, d].  causal = 1 applies the
 * square, top-left aligned mask j <= i.  sm_scale must be finite and > 0.
 * `src` must have been carved for these B, Hq, Hkv, N, d (checked against the
 * shape it records: SAGE_ERR_INVALID_ARG otherwise) and filled by
 * sage_quantize.
 */
int sage_attn_fwd_quantized(const sage_qkv_quant* src, float* out, int B, int Hq, int Hkv, int N,
                            int d, int causal, float sm_scale, void* stream);

/*
 * The whole forward pass in one call: sage_quantize into `workspace`, then
 * sage_attn_fwd_quantized.  This is the operator that replaces a model's
 * native attention (the SageAttention article presents the method as a
 * plug-and-play replacement needing no retraining; the Berkeley brief's
 * experiment steps, "落地实验标准步骤", begin by swapping the attention
 * kernel): it takes the native operator's operands -- fp16/bf16 Q, K, V in
 * [B, H, N, d], the causal flag and the softmax scale -- and returns its
 * output, in FP32.  The caller supplies the device workspace
 * (sage_workspace_bytes) so that the call never allocates.
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                  int N, int d, int causal, float sm_scale, int dtype, void* workspace,
                  size_t ws_bytes, void* stream);

/* sage_attn_fwd (E4M3 P.V) with the quantization granularity chosen by the caller:
 * (q_block, k_block) = (SAGE_BQ, SAGE_BK) is sage_attn_fwd itself,
 * (SAGE_BQ_THREAD, SAGE_BK_THREAD) the thread-level granularity,
 * (SAGE_BQ_THREAD, SAGE_BK_TOKEN) the token granularity; any other pair
 * returns SAGE_ERR_UNSUPPORTED. */
int sage_attn_fwd_granular(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                           int Hkv, int N, int d, int causal, float sm_scale, int dtype,
                           int q_block, int k_block, void* workspace, size_t ws_bytes,
                           void* stream);

/* sage_attn_fwd with every method option chosen by the caller (opts must not
 * be NULL): the quantization granularity and the P.V format.  Options outside
 * the values listed in sage_options return SAGE_ERR_UNSUPPORTED. */
int sage_attn_fwd_ex(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                     int N, int d, int causal, float sm_scale, int dtype, const sage_options* opts,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * ---- Inputs in other layouts.  A model's attention operands often come as
 * [B, N, H, d] (heads after tokens) or as views into one packed QKV tensor;
 * the operator that replaces its attention (the SageAttention article's
 * plug-and-play replacement) can read them where they lie instead of having
 * them copied into [B, H, N, d] first.
 *
 * sage_strides: the element strides (batch, head, token) of an fp16/bf16
 * [B, H, N, d] tensor whose d elements are contiguous.  [B, H, N, d] itself
 * is {H*N*d, N*d, d}; a [B, N, H, d] tensor is {N*H*d, d, H*d}.  Each
 * stride must be a non-negative multiple of 8 (every row starts 16-byte
 * aligned, as the base pointer must be), else SAGE_ERR_INVALID_ARG.  The
 * library reads element (b, h, n, c) at base + b*s.b + h*s.h + n*s.n + c and
 * nothing else; the caller guarantees those elements lie in its allocation.
 * A NULL stride pointer means the contiguous layout.  The output stays FP32
 * [B, Hq, N, d], contiguous.
 */
typedef struct {
    long long b, h, n;
} sage_strides;

/* sage_quantize with Q, K and V read through their strides.  The workspace
 * contents equal sage_quantize's on the same values, byte for byte. */
int sage_quantize_strided(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int N, int d, const sage_strides* q_strides,
                          const sage_strides* k_strides, const sage_strides* v_strides,
                          const sage_qkv_quant* dst, void* stream);

/* sage_attn_fwd_ex with Q, K and V read through their strides (opts must not
 * be NULL).  The output equals sage_attn_fwd_ex's on the same values, bit for
 * bit. */
int sage_attn_fwd_strided(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                          int Hkv, int N, int d, int causal, float sm_scale, int dtype,
                          const sage_options* opts, const sage_strides* q_strides,
                          const sage_strides* k_strides, const sage_strides* v_strides,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * ---- Short queries against a quantized KV cache (decode).
 *
 * A KV cache holds the K/V half of the prep step over Nk cached tokens,
 * quantized once: K smoothed with its channel mean over those tokens and
 * coded INT8 with one scale per k_block keys; V coded per channel, as one
 * E4M3 code byte per element (SAGE_PV_E4M3) or as binary16 (SAGE_PV_F16).
 * With E4M3 that is 2 bytes per K+V element pair instead of 4 for fp16/bf16
 * (the memory claim of the Berkeley brief's checklist).  Appending tokens
 * means quantizing the cache again: the K mean and the V scales are global
 * over the cached tokens.
 *
 * Views of a cache (filled by sage_kv_cache_carve); N_p = Nk rounded up to
 * SAGE_NPAD, rows Nk..N_p-1 zero padding:
 *   k_i8    int8 [B, Hkv, N_p, d]            codes of K - k_mean
 *   k_scale f32  [B, Hkv, N_p / k_block]
 *   k_mean  f32  [B, Hkv, d]
 *   v       [B, Hkv, N_p / SAGE_BN, d, SAGE_BN]: uint8 E4M3 codes (SAGE_PV_E4M3,
 *           V * 448 / absmax_c) or binary16 values (SAGE_PV_F16), each block's
 *           keys in the order of sage_v_key_position()
 *   v_scale f32  [B, Hkv, d]                 absmax / 448 per channel (1 with SAGE_PV_F16)
 *   v_inv, k_part, v_part, sync: working storage of sage_kv_quantize.
 */
typedef struct {
    int8_t* k_i8;
    float* k_scale;
    float* k_mean;
    void* v;
    float* v_scale;
    float* v_inv;
    double* k_part;
    float* v_part;
    int32_t* sync;
    int32_t k_block;   /* SAGE_BK or SAGE_BK_THREAD */
    int32_t pv_format; /* SAGE_PV_E4M3 or SAGE_PV_F16 */
    int32_t B, Hkv, Nk, d; /* the shape the cache was carved for (set by
                              sage_kv_cache_carve); sage_kv_quantize and
                              sage_attn_decode return SAGE_ERR_INVALID_ARG for
                              other sizes */
} sage_kv_cache;

/* Bytes of a KV cache for [B, Hkv, Nk, d] in this P.V format (0 when the
 * shape or format is invalid). */
size_t sage_kv_cache_bytes(int B, int Hkv, int Nk, int d, int pv_format);

/* Split `buf` (device memory, 256-byte aligned, `bytes` long) into the views of
 * `cache` for this K granularity (k_block = SAGE_BK or SAGE_BK_THREAD) and P.V
 * format.  Host-only; no HIP call. */
int sage_kv_cache_carve(void* buf, size_t bytes, int B, int Hkv, int Nk, int d, int k_block,
                        int pv_format, sage_kv_cache* cache);

/* The K/V half of sage_quantize: K mean, smoothing, INT8 K, V codes, from
 * fp16/bf16 K, V [B, Hkv, Nk, d] into `cache`, which must have been carved
 * for these sizes.  Runs as three kernels on `stream` (counter clearing,
 * statistics, codes). */
int sage_kv_quantize(const void* k, const void* v, int dtype, int B, int Hkv, int Nk, int d,
                     const sage_kv_cache* cache, void* stream);

/* sage_kv_quantize with K and V read through their strides (sage_strides;
 * NULL: contiguous), e.g. a cache kept as [B, Nk, Hkv, d].  The cache bytes
 * equal sage_kv_quantize's on the same values. */
int sage_kv_quantize_strided(const void* k, const void* v, int dtype, int B, int Hkv, int Nk, int d,
                             const sage_strides* k_strides, const sage_strides* v_strides,
                             const sage_kv_cache* cache, void* stream);

/* Workspace bytes sage_attn_decode needs for this shape (at least 256; 0 when
 * the shape is invalid). */
size_t sage_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * out = softmax(Q K^T sm_scale) V for a short query q [B, Hq, Nq, d]
 * (fp16/bf16, `dtype`) against the Nk keys of `cache`, as the method computes
 * it, FP32 output [B, Hq, Nq, d].  The Nq query rows sit at the last Nq of
 * the Nk positions: causal = 1 lets row i see keys j <= Nk - Nq + i (a mask
 * aligned to the bottom right; it needs Nq <= Nk), causal = 0 every key.
 * Each query row is quantized to INT8 with a scale of its own (as at the
 * thread-level granularity); the cache's k_block and pv_format apply.  The
 * key range is split into chunks whose partial results (reference max, row
 * sum, unnormalised output; a third FP32 accumulation level) are merged by a
 * second kernel in `workspace` (device memory, 256-byte aligned) when there is
 * more than one chunk.  `cache` must have been carved and quantized for these
 * B, Hkv, Nk, d (checked against the shape it records).
 */
int sage_attn_decode(const void* q, int dtype, const sage_kv_cache* cache, float* out, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, int causal, float sm_scale,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * sage_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, runtimes that forbid hipMalloc.  The
 * same arguments without the workspace: the per-chunk partials of the key
 * split go to a scratch array the library itself holds in device memory, one
 * copy per GPU, SAGE_DECODE_SCRATCH_BYTES long, kept until the process ends.
 * The call allocates nothing (the first call on a device looks the array's
 * address up, once).  Every shape sage_attn_decode accepts fits the array
 * (the key split never makes more than 32 x 1024 row-chunk partials); a shape
 * that would not returns SAGE_ERR_WORKSPACE.  Results equal sage_attn_decode's
 * bit for bit (same kernels, same partial layout).
 * All calls on one GPU share its array: calls that overlap on one GPU (two
 * streams, or two host threads without ordering) race and give undefined
 * output; serialize them (one stream, or events).
 */
#define SAGE_DECODE_SCRATCH_BYTES 17039360 /* 32 * 1024 * (128 + 2) floats, 256-byte regions */
int sage_attn_decode_noalloc(const void* q, int dtype, const sage_kv_cache* cache, float* out, int B,
                             int Hq, int Hkv, int Nq, int Nk, int d, int causal, float sm_scale,
                             void* stream);

/* Block sizes and format constants the library was compiled with. */
int sage_get_config(sage_config* c);

/* Position of key j (0 <= j < SAGE_BN) inside a block's row of v16; -1 if j
 * is out of range.  Describes the layout only (for callers that read the
 * quantized V back). */
int sage_v_key_position(int j);

/* Static, human-readable text for a sage_status value. */
const char* sage_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */
