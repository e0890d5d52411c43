// gfx950 matrix-core helpers for the KATA bf16 path.
//
// Operand layouts (16 x 16 output tiles, wave64; lane l, c16 = l % 16, g = l / 16):
//   A operand (M x K): lane l holds row c16, K-slots (g, s) s = 0..S-1
//   B operand (K x N): lane l holds column c16, the same K-slots
//   C/D accumulator  : lane l holds column c16, rows 4g + r, r = 0..3
// for v_mfma_f32_16x16x32_bf16 (S = 8) and v_mfma_f32_16x16x16_bf16 (S = 4).
// Only the pairing of A and B slots matters for the contraction, so every
// fragment below is described by its (g, s) -> K-index map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void_t;

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Split bf16 operands: a ~ hi + lo with hi = bf16(a) and lo = bf16(a - hi) (the
// difference is exact in fp32), so hi + lo carries about 16 significant bits,
// and exactly a when a is the product of two bf16 values (at most 16 significant
// bits). A product of two split operands is taken as hi*hi + hi*lo + lo*hi on
// the matrix cores (the lo*lo term is below 2^-16 of the product).
__device__ __forceinline__ uint32_t pk2_lo(float a, float b, uint32_t hi) {
    return pk2(a - lo_bf16(hi), b - hi_bf16(hi));
}
__device__ __forceinline__ void split8(const float (&f)[8], u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = pk2(f[2 * i], f[2 * i + 1]);
        lo[i] = pk2_lo(f[2 * i], f[2 * i + 1], hi[i]);
    }
}
__device__ __forceinline__ void split4(const float (&f)[4], u32x2_t& hi, u32x2_t& lo) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        hi[i] = pk2(f[2 * i], f[2 * i + 1]);
        lo[i] = pk2_lo(f[2 * i], f[2 * i + 1], hi[i]);
    }
}
// The bf16 remainder of an accumulator tile given its rounded pair words.
__device__ __forceinline__ u32x2_t lo_of(const f32x4_t& x, uint32_t h0, uint32_t h1) {
    return u32x2_t{pk2_lo(x[0], x[1], h0), pk2_lo(x[2], x[3], h1)};
}

// D = A(16x32) * B(32x16) + C with 8 bf16 per lane.
__device__ __forceinline__ f32x4_t mma32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// D = A(16x16) * B(16x16) + C with 4 bf16 per lane.
__device__ __forceinline__ f32x4_t mma16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// D = A(16x16) * B(16x16) + C issued as a 16x16x32 with the upper K half zero.
// Use it wherever a K = 16 product accumulates onto a 16x16x32 chain: feeding
// one matrix-core opcode's result to another opcode's accumulator input has
// produced stale sums on gfx950 with the wait states the compiler inserts, while
// chains of one opcode are exact.
__device__ __forceinline__ f32x4_t mma16_acc32(u32x2_t a, u32x2_t b, f32x4_t c) {
    return mma32(u32x4_t{a[0], a[1], 0u, 0u}, u32x4_t{b[0], b[1], 0u, 0u}, c);
}

// Value of lane (c16 + k) mod 16 of the same 16-lane row (DPP row rotate by
// 16 - k: row_ror:n delivers lane (c16 - n) mod 16).
template <int K>
__device__ __forceinline__ float row_fetch(float x) {
    static_assert(K > 0 && K < 16, "rotation in 1..15");
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + (16 - K), 0xf, 0xf, false));
}

// Bounded-wait-free ordering helpers for wave-private LDS buffers.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
    compiler_fence();
}

}  // namespace kata
