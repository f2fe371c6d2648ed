// Test probe: one wave runs one matrix-core instruction on operands whose
// rows (A) and columns (B) are all alike, so every output element is the
// same dot product sum_k a[k] * b[k], whatever the lanes' row and column
// assignment.  Lane half h (lanes 32h..32h+31) supplies reduction indices
// [K/2 * h, K/2 * (h + 1)) of both operands, the layout the 32x32 shapes use.
//
//   kind 0: v_mfma_f32_32x32x16_fp8_fp8         (K = 16, E4M3 bytes)
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4    (K = 64, E4M3 bytes, unit E8M0 scales)
//   kind 2: v_mfma_f32_32x32x16_f16             (K = 16, binary16 values)
//
// Used only by tests/test_gpu_fp8_matrix_core.py, to show how the FP8
// instructions sum their products.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void probe(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                            float* __restrict__ c, int kind) {
    const int l = threadIdx.x, h = l >> 5;
    v16f acc;
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    if (kind == 0) {
        const long av = *reinterpret_cast<const long*>(a + 8 * h);
        const long bv = *reinterpret_cast<const long*>(b + 8 * h);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av, bv, acc, 0, 0, 0);
    } else if (kind == 1) {
        const v8i av = *reinterpret_cast<const v8i*>(a + 32 * h);
        const v8i bv = *reinterpret_cast<const v8i*>(b + 32 * h);
        // format 0 = E4M3 for both operands; scale code 127 = 2^0
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
    } else {
        const v8h av = *reinterpret_cast<const v8h*>(a + 16 * h);
        const v8h bv = *reinterpret_cast<const v8h*>(b + 16 * h);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
    for (int v = 0; v < 16; ++v) c[l * 16 + v] = acc[v];
}

// a_host, b_host: 64 bytes each (K bytes of E4M3 codes for kinds 0 and 1, or
// 16 binary16 values for kind 2, then padding); out_host: 1024 floats (the
// 64 lanes' 16 accumulators).  Returns 0, or the HIP error code.
extern "C" int fp8_mfma_probe(const uint8_t* a_host, const uint8_t* b_host, int kind, float* out_host) {
    if (kind < 0 || kind > 2) return -1;
    uint8_t *a = nullptr, *b = nullptr;
    float* c = nullptr;
    hipError_t e = hipMalloc(&a, 64);
    if (e == hipSuccess) e = hipMalloc(&b, 64);
    if (e == hipSuccess) e = hipMalloc(&c, 1024 * sizeof(float));
    if (e == hipSuccess) e = hipMemcpy(a, a_host, 64, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(b, b_host, 64, hipMemcpyHostToDevice);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(probe, dim3(1), dim3(64), 0, 0, a, b, c, kind);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(out_host, c, 1024 * sizeof(float), hipMemcpyDeviceToHost);
    (void)hipFree(a);
    (void)hipFree(b);
    (void)hipFree(c);
    return (int)e;
}
