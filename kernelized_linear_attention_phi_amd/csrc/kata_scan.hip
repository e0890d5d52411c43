// Associative scan over chunk (or segment) states, elementwise fp32 addition.
//
// KATA explainers (gist.science, technical summary 2.3): the inter-chunk state
// is propagated by an associative scan (parallel prefix sum), cutting the
// recurrence depth over N_C chunks from O(N_C) to O(log N_C).
//
// Layout-agnostic: a "record" is E contiguous floats (one chunk's or segment's
// state). A block owns 32 consecutive elements of one sequence and walks its
// records in super-tiles of 128, each loaded at once through LDS (coalesced
// 128-byte rows, every load in flight together). Every wavefront scans one
// element across 64 records with a log2(64) = 6-step Hillis-Steele prefix on
// its 64 lanes (DPP lane shifts); 64-record tiles are chained by a running
// carry, so the depth is 6 * ceil(NR / 64) adds. The exclusive prefix is the
// inclusive one shifted by a lane (no subtraction, so a record never depends on
// its own value).
#include "kata_device.h"
#include "kata_internal.h"

namespace kata {

namespace {

constexpr int kTile = 64;      // records per wavefront scan = lanes per wavefront
constexpr int kCols = 32;      // elements per block
constexpr int kRows = 128;     // records per super-tile
constexpr int kWaves = 4;
constexpr int kColsPerWave = kCols / kWaves;

// Inclusive prefix sum over the 64 lanes of a wavefront in 6 DPP steps: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then the last lane of a row is broadcast
// into the following row(s). Lanes without a source add 0.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));  // row_shr:1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));  // row_shr:2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));  // row_shr:4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));  // row_shr:8
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));  // row_bcast:15
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}

// Lane i receives lane i-1 (lane 0 receives 0): wave_shr:1.
__device__ __forceinline__ float wave_shift_right(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x138, 0xf, 0xf, false));
}

__global__ __launch_bounds__(256) void scan_records_kernel(
    float* __restrict__ rec, int NR, int E, const float* __restrict__ init,
    float* __restrict__ total_a, float* __restrict__ total_b) {
    // a super-tile of kRows records x kCols elements is loaded with every load in
    // flight at once, scanned in LDS, and stored back
    __shared__ float tile[kRows][kCols + 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const size_t seq = blockIdx.y;
    const int e0 = blockIdx.x * kCols;
    // load/store mapping: thread -> (row phase rr = tid / kCols, column tid % kCols)
    const int lc = threadIdx.x % kCols, lr = threadIdx.x / kCols;
    constexpr int kRowStep = 256 / kCols;
    const int e = e0 + lc;
    float* base = rec + seq * (size_t)NR * E;

    // running carry of the elements this wave scans (uniform across lanes)
    float carry[kColsPerWave];
#pragma unroll
    for (int u = 0; u < kColsPerWave; ++u) {
        const int ee = e0 + wave * kColsPerWave + u;
        carry[u] = (init != nullptr && ee < E) ? init[seq * E + ee] : 0.0f;
    }

    for (int r0 = 0; r0 < NR; r0 += kRows) {
#pragma unroll
        for (int i = 0; i < kRows / kRowStep; ++i) {
            const int r = lr + kRowStep * i;
            const int rr = r0 + r;
            tile[r][lc] = (rr < NR && e < E) ? base[(size_t)rr * E + e] : 0.0f;
        }
        __syncthreads();
        // scan: lane = record, one element column at a time, 64 records per pass
#pragma unroll
        for (int h = 0; h < kRows / kTile; ++h) {
            if (r0 + h * kTile >= NR) break;
#pragma unroll
            for (int u = 0; u < kColsPerWave; ++u) {
                const int col = wave * kColsPerWave + u;
                const float inc = wave_inclusive_scan(tile[h * kTile + lane][col]);
                tile[h * kTile + lane][col] = carry[u] + wave_shift_right(inc);
                carry[u] += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kRows / kRowStep; ++i) {
            const int r = lr + kRowStep * i;
            const int rr = r0 + r;
            if (rr < NR && e < E) base[(size_t)rr * E + e] = tile[r][lc];
        }
        __syncthreads();
    }
    // inclusive totals
#pragma unroll
    for (int u = 0; u < kColsPerWave; ++u) {
        const int ee = e0 + wave * kColsPerWave + u;
        if (lane == 0 && ee < E) {
            if (total_a) total_a[seq * E + ee] = carry[u];
            if (total_b) total_b[seq * E + ee] = carry[u];
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
