// Internal definitions shared by the HIP kernels and the host side of the
// library: launch geometry, workspace layout and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/sage.h"

namespace sage {

constexpr int kThreads = 256;      // prep kernels run 4 waves of 64
constexpr int kStatRows = 512;     // rows per partial-statistics chunk of the prep step
constexpr int kVersion = 101;

// Element strides (batch, head, token) of an fp16/bf16 input whose d elements
// are contiguous; the prep step reads Q, K and V through them.
struct InStrides {
    long long b, h, n;
};

struct Shape {
    int B, Hq, Hkv, N, d;
    int Np;       // N rounded up to SAGE_NPAD
    InStrides qs, ks, vs;  // input layouts (contiguous [B, H, N, d] by default)
    long long q_elems() const { return (long long)B * Hq * Np * d; }
    long long kv_elems() const { return (long long)B * Hkv * Np * d; }
    __host__ __device__ int part_chunks() const { return (N + kStatRows - 1) / kStatRows; }
    // where head bh (b * H + h) of an input with H heads starts
    __host__ __device__ static long long head_start(const InStrides& st, int bh, int H) {
        return (long long)(bh / H) * st.b + (long long)(bh % H) * st.h;
    }
};

inline InStrides contiguous_strides(int H, int N, int d) {
    return InStrides{(long long)H * N * d, (long long)N * d, d};
}

inline Shape make_shape(int B, int Hq, int Hkv, int N, int d) {
    Shape s{B, Hq, Hkv, N, d, 0, {}, {}, {}};
    s.Np = (N + SAGE_NPAD - 1) / SAGE_NPAD * SAGE_NPAD;
    s.qs = contiguous_strides(Hq, N, d);
    s.ks = contiguous_strides(Hkv, N, d);
    s.vs = s.ks;
    return s;
}

// What the K/V half of the prep step writes, from either a full workspace
// (sage_qkv_quant) or a KV cache (sage_kv_cache).  The V operand is stored
// as the binary16 values of its E4M3 codes (the prefill workspace), as V's
// own binary16 rounding (binary16 P.V), or as E4M3 code bytes (a KV cache).
enum VStore { kVE4M3Half = 0, kVF16 = 1, kVE4M3Byte = 2 };
struct KVViews {
    int8_t* k_i8;
    float* k_scale;
    float* k_mean;
    void* v;
    float* v_scale;
    float* v_inv;
    double* k_part;
    float* v_part;
    int32_t* sync;
    int k_block;
    int v_store;
    float qmax;  // largest K code: 127 (INT8) or 7 (INT4)
};

// Split of a short-query attention over a KV cache into work-groups: row
// tiles of 32 packed (q head, query row) pairs per kv head, and chunks of
// chunk_blocks consecutive key blocks (nchunk of them).  A pure function of
// the shape, so the host can size the workspace with it.
struct DecodePlan {
    int row_tiles, nchunk, chunk_blocks;
};
// wgs_per_cu: decode work-groups resident per CU (4 by default: the most any
// configuration runs, which sizes the workspace for every format)
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int wgs_per_cu = 4);

// Position of key j inside a block's V row.  The attention kernel's 32x32
// Q.K^T tiles leave, in lane half h (lanes 32h..32h+31), the scores of keys
// 8i + 4h + j (i, j = 0..3) of each 32-key tile.  Each 16-key step of P.V
// takes 8 of them per lane as its operand elements e = 0..7, which the matrix
// core reads as reduction index 8h + e; that index belongs to key
// 8*(e/4) + 4h + e%4 of the step.  V stores each step's 16 keys in reduction
// order, so a lane reads its V operand contiguously: within every group of 16
// keys, keys 4..7 and 8..11 trade places (the map is its own inverse).
__host__ __device__ inline int v_key_position(int j) {
    const int a = (j >> 2) & 3;
    return (j & ~15) | ((((a & 1) << 1) | (a >> 1)) << 2) | (j & 3);
}

// Launch facts of one kernel on one device, settled once per (kernel, device)
// and read on every later launch without a driver call: the dynamic-LDS limit
// raised where a kernel needs more than 64 KB, and the number of its
// work-groups the device holds at once (CU count times resident work-groups
// per CU; 0 if the runtime cannot say).  `fn` is the kernel's host stub; each
// kernel instantiation passes its own LaunchFacts object.
struct LaunchFacts {
    static constexpr int kMaxDevices = 64;
    std::atomic<int> ready[kMaxDevices];
    int slots[kMaxDevices];
    hipError_t settle(const void* fn, int threads, size_t lds, int* slots_out);
};

// ---------------------------------------------------------------- device
#if defined(__HIPCC__)

template <typename T> struct In16;
template <> struct In16<_Float16> {
    static __device__ inline float to_f32(uint32_t bits16) {
        uint16_t b = (uint16_t)bits16;
        return (float)__builtin_bit_cast(_Float16, b);
    }
};
struct Bf16Tag {};
template <> struct In16<Bf16Tag> {
    static __device__ inline float to_f32(uint32_t bits16) {
        return __builtin_bit_cast(float, (bits16 & 0xFFFFu) << 16);
    }
};

// Eight 16-bit values (one 16-byte load) to float.
template <typename T>
__device__ inline void unpack8(const uint4& u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = In16<T>::to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = In16<T>::to_f32(w[i] >> 16);
    }
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// Max over the 256 threads of a block; `red` is 4 floats of shared memory.
__device__ inline float block_max(float x, float* red) {
    x = wave_max(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

#endif

}  // namespace sage
