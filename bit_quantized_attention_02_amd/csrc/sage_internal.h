// Internal definitions shared by the HIP kernels and the host side of the
// library: launch geometry, workspace layout and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sage.h"

namespace sage {

constexpr int kThreads = 256;      // prep kernels run 4 waves of 64
constexpr int kStatRows = 512;     // rows per partial-statistics chunk
constexpr int kVersion = 100;

struct Shape {
    int B, Hq, Hkv, N, d;
    int Np;       // N rounded up to SAGE_NPAD
    int nchunk;   // statistics chunks per kv head
    long long q_elems() const { return (long long)B * Hq * Np * d; }
    long long kv_elems() const { return (long long)B * Hkv * Np * d; }
};

inline Shape make_shape(int B, int Hq, int Hkv, int N, int d) {
    Shape s{B, Hq, Hkv, N, d, 0, 0};
    s.Np = (N + SAGE_NPAD - 1) / SAGE_NPAD * SAGE_NPAD;
    s.nchunk = (N + kStatRows - 1) / kStatRows;
    return s;
}

// Position of key j inside a block's V row.  After the Q.K^T product, lane
// group g (lanes 16g..16g+15) holds the scores of keys 16*tau + 4g + v
// (tau = 0..7, v = 0..3); its P.V operand element e = 4*tau + v therefore
// belongs to key 16*(e/4) + 4g + e%4, and V stores that key at position
// 32g + e, so each lane reads its V operand contiguously.
__host__ __device__ inline int v_key_position(int j) {
    int tau = j >> 4, g = (j >> 2) & 3, v = j & 3;
    return 32 * g + 4 * tau + v;
}

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
