// Device helpers shared by the KATA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
    static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void st(bf16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Packed-feature index -> (i, j), i <= j, for the row-major upper triangle:
// p(i, j) = i*d - i*(i-1)/2 + (j - i). Encoded as i | j << 8.
__device__ __forceinline__ uint32_t pack_pair(int p, int d) {
    int i = 0;
    int start = 0;
    while (start + (d - i) <= p) {
        start += d - i;
        ++i;
    }
    int j = i + (p - start);
    return static_cast<uint32_t>(i) | (static_cast<uint32_t>(j) << 8);
}

// Fills tab[0..D) with the pair codes; the caller synchronises afterwards.
__device__ __forceinline__ void fill_pair_table(uint32_t* tab, int d, int D) {
    for (int p = threadIdx.x; p < D; p += blockDim.x) tab[p] = pack_pair(p, d);
}

constexpr float kSqrt2 = 1.41421356237309504880f;

// Correctly rounded num / den with the zero-denominator rule (den == 0 -> 0).
__device__ __forceinline__ float safe_div(float num, float den) {
    return den != 0.0f ? num / den : 0.0f;
}

}  // namespace kata
