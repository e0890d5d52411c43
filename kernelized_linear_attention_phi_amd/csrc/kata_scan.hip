// Associative scan over chunk (or segment) states, elementwise fp32 addition.
//
// KATA explainers (gist.science, technical summary 2.3): the inter-chunk state
// is propagated by an associative scan (parallel prefix sum), cutting the
// recurrence depth over N_C chunks from O(N_C) to O(log N_C).
//
// Layout-agnostic: a "record" is E contiguous floats (one chunk's S or z). A
// block owns 64 consecutive elements of one sequence and walks its records in
// tiles of 64. Each tile is staged through LDS (coalesced 256-byte rows), and
// every wavefront scans one element across the 64 records of the tile with a
// log2(64) = 6-step Hillis-Steele prefix on its 64 lanes (cross-lane shuffles);
// tiles are chained by a running carry, so the depth is 6 * ceil(NR / 64) adds.
#include "kata_device.h"
#include "kata_internal.h"

namespace kata {

namespace {

constexpr int kTile = 64;      // records per tile = lanes per wavefront
constexpr int kCols = 64;      // elements per block
constexpr int kWaves = 4;
constexpr int kColsPerWave = kCols / kWaves;

__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

__global__ __launch_bounds__(256) void scan_records_kernel(
    float* __restrict__ rec, int NR, int E, const float* __restrict__ init,
    float* __restrict__ total_a, float* __restrict__ total_b) {
    __shared__ float tile[kTile][kCols + 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const size_t seq = blockIdx.y;
    const int e0 = blockIdx.x * kCols;
    float* base = rec + seq * (size_t)NR * E;

    // running carry of the elements this wave scans (uniform across lanes)
    float carry[kColsPerWave];
#pragma unroll
    for (int u = 0; u < kColsPerWave; ++u) {
        const int e = e0 + wave * kColsPerWave + u;
        carry[u] = (init != nullptr && e < E) ? init[seq * E + e] : 0.0f;
    }

    for (int r0 = 0; r0 < NR; r0 += kTile) {
        // load: wave w loads rows w, w+4, ...; lane = element (coalesced)
        for (int r = wave; r < kTile; r += kWaves) {
            const int rr = r0 + r;
            const int e = e0 + lane;
            tile[r][lane] = (rr < NR && e < E) ? base[(size_t)rr * E + e] : 0.0f;
        }
        __syncthreads();
        // scan: lane = record, one element column at a time
#pragma unroll
        for (int u = 0; u < kColsPerWave; ++u) {
            const int col = wave * kColsPerWave + u;
            const float x = tile[lane][col];
            const float inc = wave_inclusive_scan(x, lane);
            float exc = __shfl_up(inc, 1, 64);
            if (lane == 0) exc = 0.0f;
            tile[lane][col] = carry[u] + exc;
            carry[u] += __shfl(inc, 63, 64);
        }
        __syncthreads();
        for (int r = wave; r < kTile; r += kWaves) {
            const int rr = r0 + r;
            const int e = e0 + lane;
            if (rr < NR && e < E) base[(size_t)rr * E + e] = tile[r][lane];
        }
        __syncthreads();
    }
    // inclusive totals
#pragma unroll
    for (int u = 0; u < kColsPerWave; ++u) {
        const int e = e0 + wave * kColsPerWave + u;
        if (lane == 0 && e < E) {
            if (total_a) total_a[seq * E + e] = carry[u];
            if (total_b) total_b[seq * E + e] = carry[u];
        }
    }
}

__global__ void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                    size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_scan_records(float* rec, int nseq, int NR, int E, const float* init,
                               float* total_a, float* total_b, hipStream_t st) {
    if (nseq == 0 || E == 0) return hipSuccess;
    dim3 grid((E + kCols - 1) / kCols, nseq);
    scan_records_kernel<<<grid, 256, 0, st>>>(rec, NR, E, init, total_a, total_b);
    return hipGetLastError();
}

hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    copy_or_zero_kernel<<<(unsigned)blocks, 256, 0, st>>>(dst, src, n);
    return hipGetLastError();
}

}  // namespace kata
