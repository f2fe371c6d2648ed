// Host side of the C ABI declared in include/sage.h: argument validation
// (before any HIP call), workspace carving and kernel launches.
#include <math.h>
#include <string.h>

#include "sage_internal.h"

namespace sage {
hipError_t launch_prep(const void* q, const void* k, const void* v, int dtype, const Shape& s,
                       const sage_qkv_quant* z, hipStream_t st);
hipError_t launch_prep_kv(const void* k, const void* v, int dtype, const Shape& s, const KVViews& z,
                          hipStream_t st);
hipError_t launch_attn(const sage_qkv_quant* z, float* out, const Shape& s, int causal, float qk,
                       float l448, hipStream_t st);
hipError_t launch_decode(const void* q, int dtype, const sage_kv_cache* cache, float* out,
                         float* part_o, float* part_ml, int B, int Hq, int Hkv, int Nq, int Nk,
                         int d, int causal, float qk, float l448, hipStream_t st);
int prep_sync_words(const Shape& s);
}  // namespace sage

using sage::Shape;

#include <mutex>

// Serialises the first launch of a kernel on a device; later launches read
// the settled facts without locking.
static std::mutex g_launch_facts_mu;

hipError_t sage::LaunchFacts::settle(const void* fn, int threads, size_t lds, int* slots_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices && ready[dev].load(std::memory_order_acquire)) {
        *slots_out = slots[dev];
        return hipSuccess;
    }
    std::lock_guard<std::mutex> lock(g_launch_facts_mu);
    if (dev >= 0 && dev < kMaxDevices && ready[dev].load(std::memory_order_relaxed)) {
        *slots_out = slots[dev];
        return hipSuccess;
    }
    if (lds > 65536) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    int cus = 0, per_cu = 0;
    const bool known =
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) == hipSuccess;
    if (!known) (void)hipGetLastError();  // an unknown count only means "no split"
    const int n = known ? cus * per_cu : 0;
    *slots_out = n;
    if (dev >= 0 && dev < kMaxDevices) {
        slots[dev] = n;
        ready[dev].store(1, std::memory_order_release);
    }
    return hipSuccess;
}

static int check_shape(int B, int Hq, int Hkv, int N, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1) return SAGE_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
    if (Hq % Hkv != 0) return SAGE_ERR_UNSUPPORTED;
    if (N > SAGE_MAX_N) return SAGE_ERR_UNSUPPORTED;
    const Shape s = sage::make_shape(B, Hq, Hkv, N, d);
    // work-group counts must fit a 1-D grid
    if ((long long)B * Hq * (s.Np / SAGE_BQ) >= (1LL << 31)) return SAGE_ERR_UNSUPPORTED;
    // (prep_pack: K row blocks of 64, V blocks of 128 keys in up to two channel slices)
    if ((long long)B * Hkv * (s.Np / SAGE_BK + 2 * (s.Np / SAGE_BN)) >= (1LL << 31)) return SAGE_ERR_UNSUPPORTED;
    return SAGE_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: each region starts on a 256-byte boundary.  A KV cache
// (with_q false) has no Q regions, and v_bytes (1 or 2) per V element.
struct Layout {
    size_t q_i8, q_scale, k_i8, k_scale, k_mean, v16, v_scale, v_inv, k_part, v_part, sync, tail, total;
    long long tail_rows;
};

// Rows of split-tile partial results the workspace holds: at d = 64, the
// shares of up to 4096 tiles of 128 rows (a tail of several hundred tiles
// split several ways), never more than the shape's own tiles hold.
static long long tail_capacity(const Shape& s) {
    if (s.d != 64) return 0;
    const long long tiles = (long long)s.B * s.Hq * (s.Np / 128);
    return (tiles < 4096 ? tiles : 4096) * 128;
}

static Layout layout(const Shape& s, bool with_q = true, size_t v_bytes = sizeof(uint16_t)) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += round256(bytes);
        return o;
    };
    const size_t Bq = (size_t)s.B * s.Hq, Bkv = (size_t)s.B * s.Hkv;
    L.q_i8 = with_q ? take((size_t)s.q_elems()) : 0;
    L.k_i8 = take((size_t)s.kv_elems());
    L.v16 = take((size_t)s.kv_elems() * v_bytes);
    // scales sized for the finest granularity
    L.q_scale = with_q ? take(Bq * (s.Np / SAGE_BQ_THREAD) * sizeof(float)) : 0;
    L.k_scale = take(Bkv * (s.Np / SAGE_BK_TOKEN) * sizeof(float));
    L.k_mean = take(Bkv * s.d * sizeof(float));
    L.v_scale = take(Bkv * s.d * sizeof(float));
    L.v_inv = take(Bkv * s.d * sizeof(float));
    L.k_part = take(Bkv * s.part_chunks() * s.d * sizeof(double));
    L.v_part = take(Bkv * s.part_chunks() * s.d * sizeof(float));
    L.sync = take((size_t)sage::prep_sync_words(s) * sizeof(int32_t));
    L.tail_rows = with_q ? tail_capacity(s) : 0;
    L.tail = L.tail_rows ? take((size_t)L.tail_rows * (s.d + 2) * sizeof(float)) : 0;
    L.total = off;
    return L;
}

static bool granularity_ok(int q_block, int k_block) {
    return (q_block == SAGE_BQ && k_block == SAGE_BK) ||
           (q_block == SAGE_BQ_THREAD && (k_block == SAGE_BK_THREAD || k_block == SAGE_BK_TOKEN));
}

static bool pv_format_ok(int f) { return f == SAGE_PV_E4M3 || f == SAGE_PV_F16; }
static bool qk_bits_ok(int b) { return b == SAGE_QK_INT8 || b == SAGE_QK_INT4; }

static bool k_block_ok(int k_block) { return k_block == SAGE_BK || k_block == SAGE_BK_THREAD; }

// Bytes per V element of a KV cache: E4M3 codes, or binary16.
static size_t cache_v_bytes(int pv_format) { return pv_format == SAGE_PV_F16 ? 2 : 1; }

static int check_cache(const sage_kv_cache* z, int B, int Hkv, int Nk, int d) {
    if (!z) return SAGE_ERR_INVALID_ARG;
    if (z->B != B || z->Hkv != Hkv || z->Nk != Nk || z->d != d) return SAGE_ERR_INVALID_ARG;
    if (!k_block_ok(z->k_block) || !pv_format_ok(z->pv_format)) return SAGE_ERR_UNSUPPORTED;
    if (!z->k_i8 || !z->k_scale || !z->k_mean || !z->v || !z->v_scale || !z->v_inv || !z->k_part ||
        !z->v_part || !z->sync)
        return SAGE_ERR_INVALID_ARG;
    if (!aligned(z->k_i8, 16) || !aligned(z->v, 16) || !aligned(z->k_scale, 16) ||
        !aligned(z->v_scale, 16) || !aligned(z->k_part, 8))
        return SAGE_ERR_INVALID_ARG;
    return SAGE_OK;
}

// Shape of a short query (Nq rows per q head) against Nk cached keys.
static int check_decode_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (Nq < 1) return SAGE_ERR_INVALID_ARG;
    int rc = check_shape(B, Hq, Hkv, Nk, d);
    if (rc != SAGE_OK) return rc;
    if (Nq > SAGE_MAX_N) return SAGE_ERR_UNSUPPORTED;
    // query rows (and so the G * Nq packed rows of a kv head) fit an int
    // before the plan is formed from them
    if ((long long)B * Hq * Nq >= (1LL << 31)) return SAGE_ERR_UNSUPPORTED;
    const sage::DecodePlan pl = sage::decode_plan(B, Hq, Hkv, Nq, Nk, d);
    if ((long long)B * Hkv * pl.nchunk * pl.row_tiles >= (1LL << 31)) return SAGE_ERR_UNSUPPORTED;
    return SAGE_OK;
}

// Decode workspace: the per-chunk partials, (rows x chunks x d) and
// (rows x chunks x 2) floats; at least 256 bytes so that 0 means "invalid".
struct DecodeLayout {
    size_t part_o, part_ml, total;
};

static DecodeLayout decode_layout(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    const sage::DecodePlan pl = sage::decode_plan(B, Hq, Hkv, Nq, Nk, d);
    DecodeLayout L;
    const size_t parts = pl.nchunk > 1 ? (size_t)B * Hq * Nq * pl.nchunk : 0;
    L.part_o = 0;
    L.part_ml = round256(parts * d * sizeof(float));
    L.total = L.part_ml + round256(parts * 2 * sizeof(float));
    if (L.total < 256) L.total = 256;
    return L;
}

// The views are read and written by the sizes a call is passed: they must be
// the sizes the struct was carved for.
static int check_quant(const sage_qkv_quant* z, int B, int Hq, int Hkv, int N, int d) {
    if (!z) return SAGE_ERR_INVALID_ARG;
    if (z->B != B || z->Hq != Hq || z->Hkv != Hkv || z->N != N || z->d != d) return SAGE_ERR_INVALID_ARG;
    if (!granularity_ok(z->q_block, z->k_block) || !pv_format_ok(z->pv_format) ||
        !qk_bits_ok(z->qk_bits))
        return SAGE_ERR_UNSUPPORTED;
    if (!z->q_i8 || !z->q_scale || !z->k_i8 || !z->k_scale || !z->k_mean || !z->v16 ||
        !z->v_scale || !z->v_inv || !z->k_part || !z->v_part || !z->sync)
        return SAGE_ERR_INVALID_ARG;
    if (!aligned(z->q_i8, 16) || !aligned(z->k_i8, 16) || !aligned(z->v16, 16) ||
        !aligned(z->v_scale, 16) || !aligned(z->k_part, 8))
        return SAGE_ERR_INVALID_ARG;
    if (z->tail_rows < 0 || (z->tail_part && !aligned(z->tail_part, 16))) return SAGE_ERR_INVALID_ARG;
    return SAGE_OK;
}

extern "C" {

size_t sage_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
    if (check_shape(B, Hq, Hkv, N, d) != SAGE_OK) return 0;
    return layout(sage::make_shape(B, Hq, Hkv, N, d)).total;
}

int sage_workspace_carve(void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int N, int d,
                         sage_qkv_quant* out) {
    int rc = check_shape(B, Hq, Hkv, N, d);
    if (rc != SAGE_OK) return rc;
    if (!out) return SAGE_ERR_INVALID_ARG;
    if (!ws || !aligned(ws, 256)) return SAGE_ERR_WORKSPACE;
    const Layout L = layout(sage::make_shape(B, Hq, Hkv, N, d));
    if (ws_bytes < L.total) return SAGE_ERR_WORKSPACE;
    char* base = (char*)ws;
    out->q_i8 = (int8_t*)(base + L.q_i8);
    out->q_scale = (float*)(base + L.q_scale);
    out->k_i8 = (int8_t*)(base + L.k_i8);
    out->k_scale = (float*)(base + L.k_scale);
    out->k_mean = (float*)(base + L.k_mean);
    out->v16 = (uint16_t*)(base + L.v16);
    out->v_scale = (float*)(base + L.v_scale);
    out->v_inv = (float*)(base + L.v_inv);
    out->k_part = (double*)(base + L.k_part);
    out->v_part = (float*)(base + L.v_part);
    out->sync = (int32_t*)(base + L.sync);
    out->tail_part = L.tail_rows ? (float*)(base + L.tail) : nullptr;
    out->tail_rows = L.tail_rows;
    out->q_block = SAGE_BQ;
    out->k_block = SAGE_BK;
    out->pv_format = SAGE_PV_E4M3;
    out->qk_bits = SAGE_QK_INT8;
    out->B = B;
    out->Hq = Hq;
    out->Hkv = Hkv;
    out->N = N;
    out->d = d;
    return SAGE_OK;
}

// An input layout from the caller's strides (NULL: contiguous).  Every row
// must start 16 bytes apart from the base in multiples (the prep step reads
// 16-byte pieces), so each stride is a non-negative multiple of 8 elements.
static bool take_strides(const sage_strides* st, sage::InStrides* out) {
    if (!st) return true;
    if (st->b < 0 || st->h < 0 || st->n < 0 || st->b % 8 || st->h % 8 || st->n % 8) return false;
    *out = sage::InStrides{st->b, st->h, st->n};
    return true;
}

static int quantize_impl(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                         int N, int d, const sage_strides* qst, const sage_strides* kst,
                         const sage_strides* vst, const sage_qkv_quant* dst, void* stream) {
    int rc = check_shape(B, Hq, Hkv, N, d);
    if (rc != SAGE_OK) return rc;
    if (dtype != SAGE_F16 && dtype != SAGE_BF16) return SAGE_ERR_INVALID_ARG;
    if (!q || !k || !v || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return SAGE_ERR_INVALID_ARG;
    Shape s = sage::make_shape(B, Hq, Hkv, N, d);
    if (!take_strides(qst, &s.qs) || !take_strides(kst, &s.ks) || !take_strides(vst, &s.vs))
        return SAGE_ERR_INVALID_ARG;
    rc = check_quant(dst, B, Hq, Hkv, N, d);
    if (rc != SAGE_OK) return rc;
    hipError_t e = sage::launch_prep(q, k, v, dtype, s, dst, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_quantize(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                  int N, int d, const sage_qkv_quant* dst, void* stream) {
    return quantize_impl(q, k, v, dtype, B, Hq, Hkv, N, d, nullptr, nullptr, nullptr, dst, stream);
}

int sage_quantize_strided(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int N, int d, const sage_strides* q_strides,
                          const sage_strides* k_strides, const sage_strides* v_strides,
                          const sage_qkv_quant* dst, void* stream) {
    return quantize_impl(q, k, v, dtype, B, Hq, Hkv, N, d, q_strides, k_strides, v_strides, dst, stream);
}

int sage_attn_fwd_quantized(const sage_qkv_quant* src, float* out, int B, int Hq, int Hkv, int N,
                            int d, int causal, float sm_scale, void* stream) {
    int rc = check_shape(B, Hq, Hkv, N, d);
    if (rc != SAGE_OK) return rc;
    if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
    if (!(sm_scale > 0.0f) || !isfinite(sm_scale)) return SAGE_ERR_INVALID_ARG;
    if (!out || !aligned(out, 16)) return SAGE_ERR_INVALID_ARG;
    rc = check_quant(src, B, Hq, Hkv, N, d);
    if (rc != SAGE_OK) return rc;
    const Shape s = sage::make_shape(B, Hq, Hkv, N, d);
    // the exponent factor and log2 of the P block maximum's code (448 for
    // E4M3, 1 for binary16) are rounded once to float32 here, as the method's
    // spec defines them
    const float qk = (float)((double)sm_scale * 1.4426950408889634);
    const float l448 = src->pv_format == SAGE_PV_F16 ? 0.0f : (float)log2(448.0);
    hipError_t e = sage::launch_attn(src, out, s, causal, qk, l448, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

static int attn_fwd_impl(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                         int N, int d, int causal, float sm_scale, int dtype, const sage_options* opts,
                         const sage_strides* qst, const sage_strides* kst, const sage_strides* vst,
                         void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_shape(B, Hq, Hkv, N, d);
    if (rc != SAGE_OK) return rc;
    if (!opts) return SAGE_ERR_INVALID_ARG;
    if (!granularity_ok(opts->q_block, opts->k_block) || !pv_format_ok(opts->pv_format) ||
        !qk_bits_ok(opts->qk_bits))
        return SAGE_ERR_UNSUPPORTED;
    if (dtype != SAGE_F16 && dtype != SAGE_BF16) return SAGE_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
    if (!(sm_scale > 0.0f) || !isfinite(sm_scale)) return SAGE_ERR_INVALID_ARG;
    if (!q || !k || !v || !out || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(out, 16))
        return SAGE_ERR_INVALID_ARG;
    sage_qkv_quant z;
    rc = sage_workspace_carve(workspace, ws_bytes, B, Hq, Hkv, N, d, &z);
    if (rc != SAGE_OK) return rc;
    z.q_block = opts->q_block;
    z.k_block = opts->k_block;
    z.pv_format = opts->pv_format;
    z.qk_bits = opts->qk_bits;
    rc = quantize_impl(q, k, v, dtype, B, Hq, Hkv, N, d, qst, kst, vst, &z, stream);
    if (rc != SAGE_OK) return rc;
    return sage_attn_fwd_quantized(&z, out, B, Hq, Hkv, N, d, causal, sm_scale, stream);
}

int sage_attn_fwd_ex(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                     int N, int d, int causal, float sm_scale, int dtype, const sage_options* opts,
                     void* workspace, size_t ws_bytes, void* stream) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, N, d, causal, sm_scale, dtype, opts, nullptr, nullptr,
                         nullptr, workspace, ws_bytes, stream);
}

int sage_attn_fwd_strided(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                          int Hkv, int N, int d, int causal, float sm_scale, int dtype,
                          const sage_options* opts, const sage_strides* q_strides,
                          const sage_strides* k_strides, const sage_strides* v_strides,
                          void* workspace, size_t ws_bytes, void* stream) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, N, d, causal, sm_scale, dtype, opts, q_strides, k_strides,
                         v_strides, workspace, ws_bytes, stream);
}

int sage_attn_fwd_granular(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                           int Hkv, int N, int d, int causal, float sm_scale, int dtype,
                           int q_block, int k_block, void* workspace, size_t ws_bytes,
                           void* stream) {
    const sage_options o = {q_block, k_block, SAGE_PV_E4M3, SAGE_QK_INT8};
    return sage_attn_fwd_ex(q, k, v, out, B, Hq, Hkv, N, d, causal, sm_scale, dtype, &o, workspace,
                            ws_bytes, stream);
}

int sage_attn_fwd(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                  int N, int d, int causal, float sm_scale, int dtype, void* workspace,
                  size_t ws_bytes, void* stream) {
    return sage_attn_fwd_granular(q, k, v, out, B, Hq, Hkv, N, d, causal, sm_scale, dtype, SAGE_BQ,
                                  SAGE_BK, workspace, ws_bytes, stream);
}

size_t sage_kv_cache_bytes(int B, int Hkv, int Nk, int d, int pv_format) {
    if (check_shape(B, Hkv, Hkv, Nk, d) != SAGE_OK || !pv_format_ok(pv_format)) return 0;
    return layout(sage::make_shape(B, Hkv, Hkv, Nk, d), false, cache_v_bytes(pv_format)).total;
}

int sage_kv_cache_carve(void* buf, size_t bytes, int B, int Hkv, int Nk, int d, int k_block,
                        int pv_format, sage_kv_cache* out) {
    int rc = check_shape(B, Hkv, Hkv, Nk, d);
    if (rc != SAGE_OK) return rc;
    if (!k_block_ok(k_block) || !pv_format_ok(pv_format)) return SAGE_ERR_UNSUPPORTED;
    if (!out) return SAGE_ERR_INVALID_ARG;
    if (!buf || !aligned(buf, 256)) return SAGE_ERR_WORKSPACE;
    const Layout L = layout(sage::make_shape(B, Hkv, Hkv, Nk, d), false, cache_v_bytes(pv_format));
    if (bytes < L.total) return SAGE_ERR_WORKSPACE;
    char* base = (char*)buf;
    out->k_i8 = (int8_t*)(base + L.k_i8);
    out->k_scale = (float*)(base + L.k_scale);
    out->k_mean = (float*)(base + L.k_mean);
    out->v = (void*)(base + L.v16);
    out->v_scale = (float*)(base + L.v_scale);
    out->v_inv = (float*)(base + L.v_inv);
    out->k_part = (double*)(base + L.k_part);
    out->v_part = (float*)(base + L.v_part);
    out->sync = (int32_t*)(base + L.sync);
    out->k_block = k_block;
    out->pv_format = pv_format;
    out->B = B;
    out->Hkv = Hkv;
    out->Nk = Nk;
    out->d = d;
    return SAGE_OK;
}

static int kv_quantize_impl(const void* k, const void* v, int dtype, int B, int Hkv, int Nk, int d,
                            const sage_strides* kst, const sage_strides* vst, const sage_kv_cache* cache,
                            void* stream) {
    int rc = check_shape(B, Hkv, Hkv, Nk, d);
    if (rc != SAGE_OK) return rc;
    if (dtype != SAGE_F16 && dtype != SAGE_BF16) return SAGE_ERR_INVALID_ARG;
    if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return SAGE_ERR_INVALID_ARG;
    Shape s = sage::make_shape(B, Hkv, Hkv, Nk, d);
    if (!take_strides(kst, &s.ks) || !take_strides(vst, &s.vs)) return SAGE_ERR_INVALID_ARG;
    rc = check_cache(cache, B, Hkv, Nk, d);
    if (rc != SAGE_OK) return rc;
    const sage::KVViews kv = {cache->k_i8,   cache->k_scale, cache->k_mean, cache->v,
                              cache->v_scale, cache->v_inv,  cache->k_part, cache->v_part,
                              cache->sync,   cache->k_block,
                              cache->pv_format == SAGE_PV_F16 ? sage::kVF16 : sage::kVE4M3Byte,
                              127.0f};
    hipError_t e = sage::launch_prep_kv(k, v, dtype, s, kv, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_kv_quantize(const void* k, const void* v, int dtype, int B, int Hkv, int Nk, int d,
                     const sage_kv_cache* cache, void* stream) {
    return kv_quantize_impl(k, v, dtype, B, Hkv, Nk, d, nullptr, nullptr, cache, stream);
}

int sage_kv_quantize_strided(const void* k, const void* v, int dtype, int B, int Hkv, int Nk, int d,
                             const sage_strides* k_strides, const sage_strides* v_strides,
                             const sage_kv_cache* cache, void* stream) {
    return kv_quantize_impl(k, v, dtype, B, Hkv, Nk, d, k_strides, v_strides, cache, stream);
}

size_t sage_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (check_decode_shape(B, Hq, Hkv, Nq, Nk, d) != SAGE_OK) return 0;
    return decode_layout(B, Hq, Hkv, Nq, Nk, d).total;
}

// ---- The scratch of sage_attn_decode_noalloc: the decode key split's
// per-chunk partials (part_o then part_ml, as in a decode workspace) in a
// file-scope device array, one copy per GPU.  Its host-side name is only a
// stand-in; the device address of each GPU's copy is looked up once, with that
// device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[SAGE_DECODE_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static std::atomic<void*> g_scratch_ptr[sage::LaunchFacts::kMaxDevices];

static int scratch_of_current_device(char** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
    if (dev < 0 || dev >= sage::LaunchFacts::kMaxDevices) return SAGE_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return SAGE_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = (char*)p;
    return SAGE_OK;
}

// Validation shared by the two decode entry points (host only, no HIP call).
static int check_decode_call(const void* q, int dtype, const sage_kv_cache* cache, const float* out,
                             int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                             float sm_scale) {
    int rc = check_decode_shape(B, Hq, Hkv, Nq, Nk, d);
    if (rc != SAGE_OK) return rc;
    if (dtype != SAGE_F16 && dtype != SAGE_BF16) return SAGE_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return SAGE_ERR_INVALID_ARG;
    if (!(sm_scale > 0.0f) || !isfinite(sm_scale)) return SAGE_ERR_INVALID_ARG;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return SAGE_ERR_INVALID_ARG;
    return check_cache(cache, B, Hkv, Nk, d);
}

static hipError_t run_decode(const void* q, int dtype, const sage_kv_cache* cache, float* out,
                             char* base, const DecodeLayout& L, int B, int Hq, int Hkv, int Nq,
                             int Nk, int d, int causal, float sm_scale, void* stream) {
    const float qk = (float)((double)sm_scale * 1.4426950408889634);
    const float l448 = cache->pv_format == SAGE_PV_F16 ? 0.0f : (float)log2(448.0);
    return sage::launch_decode(q, dtype, cache, out, (float*)(base + L.part_o),
                               (float*)(base + L.part_ml), B, Hq, Hkv, Nq, Nk, d, causal, qk, l448,
                               (hipStream_t)stream);
}

int sage_attn_decode(const void* q, int dtype, const sage_kv_cache* cache, float* out, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, int causal, float sm_scale,
                     void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_decode_call(q, dtype, cache, out, B, Hq, Hkv, Nq, Nk, d, causal, sm_scale);
    if (rc != SAGE_OK) return rc;
    const DecodeLayout L = decode_layout(B, Hq, Hkv, Nq, Nk, d);
    if (!workspace || !aligned(workspace, 256) || ws_bytes < L.total) return SAGE_ERR_WORKSPACE;
    hipError_t e = run_decode(q, dtype, cache, out, (char*)workspace, L, B, Hq, Hkv, Nq, Nk, d, causal,
                              sm_scale, stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_attn_decode_noalloc(const void* q, int dtype, const sage_kv_cache* cache, float* out, int B,
                             int Hq, int Hkv, int Nq, int Nk, int d, int causal, float sm_scale,
                             void* stream) {
    int rc = check_decode_call(q, dtype, cache, out, B, Hq, Hkv, Nq, Nk, d, causal, sm_scale);
    if (rc != SAGE_OK) return rc;
    const DecodeLayout L = decode_layout(B, Hq, Hkv, Nq, Nk, d);
    if (L.total > (size_t)SAGE_DECODE_SCRATCH_BYTES) return SAGE_ERR_WORKSPACE;
    char* base = nullptr;
    rc = scratch_of_current_device(&base);
    if (rc != SAGE_OK) return rc;
    hipError_t e = run_decode(q, dtype, cache, out, base, L, B, Hq, Hkv, Nq, Nk, d, causal, sm_scale,
                              stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_get_config(sage_config* c) {
    if (!c) return SAGE_ERR_INVALID_ARG;
    c->bq = SAGE_BQ;
    c->bk = SAGE_BK;
    c->bn = SAGE_BN;
    c->fp8_max = SAGE_FP8_MAX;
    c->version = sage::kVersion;
    return SAGE_OK;
}

int sage_v_key_position(int j) {
    if (j < 0 || j >= SAGE_BN) return -1;
    return sage::v_key_position(j);
}

const char* sage_status_string(int status) {
    switch (status) {
        case SAGE_OK: return "ok";
        case SAGE_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad flag or size)";
        case SAGE_ERR_UNSUPPORTED:
            return "unsupported shape or option (d must be 64 or 128, Hq % Hkv == 0, N <= 2^20; "
                   "(q_block, k_block) = (128, 64), (1, 32) or (1, 1); P.V format E4M3 (0) or binary16 (1); "
                   "Q, K codes of 8 or 4 bits)";
        case SAGE_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
        case SAGE_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
