// Host-side exercise of every entry point of include/sage.h, for a build of
// the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizers.py).  Every call here either needs no device
// (sizes, layouts, introspection) or is rejected by the host-side validation
// before any HIP call, so the program runs without a GPU; the device pointers
// it passes are never dereferenced.  Exit status 0: every call returned what
// it should; the sanitizers report anything else they see on stderr.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/sage.h"

static int failures = 0;

static void expect(bool ok, const char* what, int line) {
    if (!ok) {
        fprintf(stderr, "abi_driver: line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

static void* const fake = (void*)(uintptr_t(1) << 40);  // 256-byte aligned, never touched

int main() {
    // ---- introspection
    sage_config cfg;
    EXPECT(sage_get_config(&cfg) == SAGE_OK);
    EXPECT(sage_get_config(nullptr) < 0);
    for (int st = -10; st <= 10; ++st) EXPECT(sage_status_string(st) != nullptr);
    for (int j = -5; j < 200; ++j) {
        const int p = sage_v_key_position(j);
        EXPECT((j >= 0 && j < SAGE_BN) ? (p >= 0 && p < SAGE_BN) : p == -1);
    }

    // ---- sizes over a grid that reaches the limits (32-bit products would
    // overflow at the large ones)
    const int Bs[] = {1, 7, 1 << 10, 1 << 20, -1, 0};
    const int Hs[][2] = {{1, 1}, {32, 8}, {30, 30}, {3, 2}, {0, 1}, {1 << 12, 1 << 10}};
    const int Ns[] = {1, 255, 256, 4097, 17550, 1 << 20, (1 << 20) + 1, 0, -3};
    const int ds[] = {64, 128, 96, 0};
    for (int B : Bs)
        for (auto& H : Hs)
            for (int N : Ns)
                for (int d : ds) {
                    const size_t ws = sage_workspace_bytes(B, H[0], H[1], N, d);
                    const bool valid = B >= 1 && H[0] >= 1 && H[1] >= 1 && H[0] % H[1] == 0 && N >= 1 &&
                                       N <= SAGE_MAX_N && (d == 64 || d == 128);
                    if (!valid) EXPECT(ws == 0);
                    (void)sage_kv_cache_bytes(B, H[1], N, d, SAGE_PV_E4M3);
                    (void)sage_kv_cache_bytes(B, H[1], N, d, SAGE_PV_F16);
                    (void)sage_kv_cache_bytes(B, H[1], N, d, 7);
                    for (int Nq : {1, 3, 16, N, N + 1})
                        (void)sage_decode_workspace_bytes(B, H[0], H[1], Nq, N, d);
                }

    // ---- workspace carving (host arithmetic only)
    const int B = 1, Hq = 4, Hkv = 2, N = 300, d = 64;
    const size_t need = sage_workspace_bytes(B, Hq, Hkv, N, d);
    EXPECT(need > 0);
    sage_qkv_quant z;
    memset(&z, 0, sizeof z);
    EXPECT(sage_workspace_carve(fake, need, B, Hq, Hkv, N, d, &z) == SAGE_OK);
    EXPECT(sage_workspace_carve(fake, need - 1, B, Hq, Hkv, N, d, &z) < 0);
    EXPECT(sage_workspace_carve((char*)fake + 16, need, B, Hq, Hkv, N, d, &z) < 0);
    EXPECT(sage_workspace_carve(nullptr, need, B, Hq, Hkv, N, d, &z) < 0);
    EXPECT(sage_workspace_carve(fake, need, B, Hq, Hkv, N, 80, &z) < 0);
    EXPECT(sage_workspace_carve(fake, need, B, Hq, Hkv, N, d, nullptr) < 0);
    EXPECT(sage_workspace_carve(fake, need, B, Hq, Hkv, N, d, &z) == SAGE_OK);

    float* const out = (float*)fake;
    const float sm = 0.125f;
    // ---- sage_attn_fwd: every argument wrong in turn
    EXPECT(sage_attn_fwd(nullptr, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out + 1, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, (char*)fake + 2, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, fake, need,
                         nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 2, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, 5, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, 0.0f, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, NAN, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, INFINITY, SAGE_F16, fake, need,
                         nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, 96, 0, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, 3, Hkv, N, d, 0, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, 0, d, 0, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, -1, Hq, Hkv, N, d, 0, sm, SAGE_F16, fake, need, nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, fake, need - 256, nullptr) <
           0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, (char*)fake + 128, need,
                         nullptr) < 0);
    EXPECT(sage_attn_fwd(fake, fake, fake, out, B, Hq, Hkv, (1 << 20) + 1, d, 0, sm, SAGE_F16, fake, need,
                         nullptr) < 0);

    // ---- granularity, P.V format and code width
    const int grans[][3] = {{128, 64, 1}, {1, 32, 1}, {1, 1, 1}, {1, 64, 0}, {128, 32, 0}, {32, 32, 0},
                            {0, 0, 0}, {-1, 1, 0}};
    for (auto& g : grans) {
        // valid pairs get as far as the null output pointer
        EXPECT(sage_attn_fwd_granular(fake, fake, fake, nullptr, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, g[0], g[1],
                                      fake, need, nullptr) < 0);
        for (int pv : {0, 1, 2, -1})
            for (int bits : {8, 4, 5, 0}) {
                sage_options o;
                o.q_block = g[0];
                o.k_block = g[1];
                o.pv_format = pv;
                o.qk_bits = bits;
                EXPECT(sage_attn_fwd_ex(fake, fake, fake, nullptr, B, Hq, Hkv, N, d, 0, sm, SAGE_BF16, &o, fake,
                                        need, nullptr) < 0);
                sage_qkv_quant zz = z;
                zz.q_block = g[0];
                zz.k_block = g[1];
                zz.pv_format = pv;
                zz.qk_bits = bits;
                // a null input, or a recorded shape other than the call's
                EXPECT(sage_quantize(fake, nullptr, fake, SAGE_F16, B, Hq, Hkv, N, d, &zz, nullptr) < 0);
                EXPECT(sage_attn_fwd_quantized(&zz, out, B, Hq, Hkv, N + 1, d, 0, sm, nullptr) < 0);
                EXPECT(sage_attn_fwd_quantized(&zz, nullptr, B, Hq, Hkv, N, d, 0, sm, nullptr) < 0);
            }
    }
    EXPECT(sage_attn_fwd_ex(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, nullptr, fake, need,
                            nullptr) < 0);
    EXPECT(sage_quantize(fake, fake, fake, SAGE_F16, B, Hq, Hkv, N, d, nullptr, nullptr) < 0);
    EXPECT(sage_quantize(fake, fake, fake, 3, B, Hq, Hkv, N, d, &z, nullptr) < 0);
    EXPECT(sage_quantize(fake, fake, fake, SAGE_F16, B, Hq, Hkv, N, 192, &z, nullptr) < 0);
    {
        sage_qkv_quant bad = z;
        bad.v16 = nullptr;
        EXPECT(sage_quantize(fake, fake, fake, SAGE_F16, B, Hq, Hkv, N, d, &bad, nullptr) < 0);
    }
    // ---- strided inputs: bad strides in each slot, and the contiguous calls' checks
    {
        const sage_strides bad[] = {{4, 64, 256}, {8, 12, 256}, {-8, 64, 256}, {8, 64, 260}, {1LL << 40 | 4, 64, 256}};
        const sage_strides good = {(long long)N * Hq * d, d, (long long)Hq * d};
        sage_options o = {SAGE_BQ, SAGE_BK, SAGE_PV_E4M3, SAGE_QK_INT8};
        for (const auto& b : bad)
            for (int slot = 0; slot < 3; ++slot) {
                const sage_strides* st[3] = {nullptr, nullptr, nullptr};
                st[slot] = &b;
                EXPECT(sage_quantize_strided(fake, fake, fake, SAGE_F16, B, Hq, Hkv, N, d, st[0], st[1], st[2], &z,
                                             nullptr) == SAGE_ERR_INVALID_ARG);
                EXPECT(sage_attn_fwd_strided(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, &o, st[0],
                                             st[1], st[2], fake, need, nullptr) == SAGE_ERR_INVALID_ARG);
            }
        EXPECT(sage_quantize_strided(nullptr, fake, fake, SAGE_F16, B, Hq, Hkv, N, d, &good, nullptr, nullptr, &z,
                                     nullptr) < 0);
        EXPECT(sage_quantize_strided(fake, fake, fake, SAGE_F16, B, Hq, Hkv, N, d, &good, nullptr, nullptr,
                                     nullptr, nullptr) < 0);
        EXPECT(sage_attn_fwd_strided(fake, fake, fake, out, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, nullptr, &good,
                                     nullptr, nullptr, fake, need, nullptr) < 0);
        EXPECT(sage_attn_fwd_strided(fake, fake, fake, nullptr, B, Hq, Hkv, N, d, 0, sm, SAGE_F16, &o, &good,
                                     &good, nullptr, fake, need, nullptr) < 0);
        // a KV cache from strided K, V: bad strides, and a cache not carved for the shape
        const size_t cneed = sage_kv_cache_bytes(B, Hkv, N, d, SAGE_PV_E4M3);
        sage_kv_cache kc;
        EXPECT(sage_kv_cache_carve(fake, cneed, B, Hkv, N, d, SAGE_BK, SAGE_PV_E4M3, &kc) == SAGE_OK);
        for (const auto& b : bad) {
            EXPECT(sage_kv_quantize_strided(fake, fake, SAGE_F16, B, Hkv, N, d, &b, nullptr, &kc, nullptr) ==
                   SAGE_ERR_INVALID_ARG);
            EXPECT(sage_kv_quantize_strided(fake, fake, SAGE_F16, B, Hkv, N, d, nullptr, &b, &kc, nullptr) ==
                   SAGE_ERR_INVALID_ARG);
        }
        EXPECT(sage_kv_quantize_strided(fake, fake, SAGE_F16, B, Hkv, N + 1, d, &good, &good, &kc, nullptr) < 0);
        EXPECT(sage_kv_quantize_strided(fake, fake, SAGE_F16, B, Hkv, N, d, &good, &good, nullptr, nullptr) < 0);
    }
    EXPECT(sage_attn_fwd_quantized(nullptr, out, B, Hq, Hkv, N, d, 0, sm, nullptr) < 0);
    EXPECT(sage_attn_fwd_quantized(&z, out, B, Hq, Hkv, N, d, -1, sm, nullptr) < 0);
    EXPECT(sage_attn_fwd_quantized(&z, out, B, Hq, Hkv, N, d, 0, -1.0f, nullptr) < 0);

    // ---- KV cache and decode
    const int Nk = 5000, Nq = 3;
    for (int pv : {SAGE_PV_E4M3, SAGE_PV_F16}) {
        const size_t cb = sage_kv_cache_bytes(B, Hkv, Nk, d, pv);
        EXPECT(cb > 0);
        sage_kv_cache c;
        memset(&c, 0, sizeof c);
        EXPECT(sage_kv_cache_carve(fake, cb, B, Hkv, Nk, d, SAGE_BK, pv, &c) == SAGE_OK);
        EXPECT(sage_kv_cache_carve(fake, cb - 1, B, Hkv, Nk, d, SAGE_BK, pv, &c) < 0);
        EXPECT(sage_kv_cache_carve(fake, cb, B, Hkv, Nk, d, 7, pv, &c) < 0);
        EXPECT(sage_kv_cache_carve(fake, cb, B, Hkv, Nk, d, SAGE_BK, 9, &c) < 0);
        EXPECT(sage_kv_cache_carve((char*)fake + 8, cb, B, Hkv, Nk, d, SAGE_BK, pv, &c) < 0);
        EXPECT(sage_kv_cache_carve(fake, cb, B, Hkv, Nk, d, SAGE_BK_THREAD, pv, &c) == SAGE_OK);
        EXPECT(sage_kv_quantize(nullptr, fake, SAGE_BF16, B, Hkv, Nk, d, &c, nullptr) < 0);
        EXPECT(sage_kv_quantize(fake, fake, SAGE_BF16, B, Hkv, Nk + 1, d, &c, nullptr) < 0);
        EXPECT(sage_kv_quantize(fake, fake, 4, B, Hkv, Nk, d, &c, nullptr) < 0);
        EXPECT(sage_kv_quantize(fake, fake, SAGE_BF16, B, Hkv, Nk, d, nullptr, nullptr) < 0);
        const size_t dw = sage_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d);
        EXPECT(dw > 0);
        EXPECT(sage_attn_decode(nullptr, SAGE_BF16, &c, out, B, Hq, Hkv, Nq, Nk, d, 1, sm, fake, dw, nullptr) <
               0);
        EXPECT(sage_attn_decode(fake, SAGE_BF16, &c, out, B, Hq, Hkv, Nq, Nk, d, 1, sm, fake, dw - 256,
                                nullptr) < 0);
        EXPECT(sage_attn_decode(fake, SAGE_BF16, &c, out, B, Hq, Hkv, Nk + 1, Nk, d, 1, sm, fake, dw,
                                nullptr) < 0);
        EXPECT(sage_attn_decode(fake, SAGE_BF16, &c, out, B, Hq, Hkv, Nq, Nk - 1, d, 1, sm, fake, dw,
                                nullptr) < 0);
        EXPECT(sage_attn_decode(fake, SAGE_BF16, nullptr, out, B, Hq, Hkv, Nq, Nk, d, 1, sm, fake, dw,
                                nullptr) < 0);
        EXPECT(sage_attn_decode_noalloc(fake, SAGE_BF16, &c, nullptr, B, Hq, Hkv, Nq, Nk, d, 1, sm, nullptr) <
               0);
        EXPECT(sage_attn_decode_noalloc(fake, SAGE_BF16, &c, out, B, Hq, Hkv, Nq, Nk, d, 3, sm, nullptr) < 0);
        EXPECT(sage_attn_decode_noalloc(fake, SAGE_BF16, &c, out, B, Hq, Hkv, Nq, Nk, d, 1, NAN, nullptr) <
               0);
        EXPECT(sage_attn_decode_noalloc(fake, SAGE_BF16, &c, out, 1 << 20, Hq, Hkv, Nq, 1 << 20, d, 1, sm,
                                        nullptr) < 0);
    }

    if (failures) {
        fprintf(stderr, "abi_driver: %d unexpected results\n", failures);
        return 1;
    }
    printf("abi_driver: all calls returned as expected\n");
    return 0;
}
