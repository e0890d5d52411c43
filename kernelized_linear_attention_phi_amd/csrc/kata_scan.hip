// Associative scan over chunk (or segment) states, elementwise fp32 addition.
//
// KATA explainers (gist.science, technical summary 2.3): the inter-chunk state
// is propagated by an associative scan (parallel prefix sum) over chunk states
// instead of a sequential recurrence.
//
// Layout-agnostic: a "record" is E contiguous floats (one chunk's or segment's
// state; E is a multiple of 4). Optionally the inclusive total is also written
// straight to the packed state of the boundary (the record layout named by the
// caller, kata_records.h), which saves a conversion pass after the scan. The scan is exclusive: record r becomes
// init + sum_{r' < r} rec_{r'}, and the inclusive total goes to the totals.
// Sequences of at most 32 records take a per-element walk; longer ones a
// blocked two-level scan: groups of 16 consecutive records are summed in
// parallel, the group sums are prefixed, and each group is walked from its
// offset. Either way each record is read once and written once, with many
// 16-byte loads in flight per thread, since the scan is bound by HBM.
//
// Decay-gated variant: record r also carries the factor a_r by which its span
// decays the state before it, and the operator becomes
// (a1, S1) o (a2, S2) = (a1 a2, a2 S1 + S2) (1 earlier): associative but not
// commutative, so the walk is carry <- a_r carry + S_r and group aggregates are
// combined in order.
#include "kata_device.h"
#include "kata_internal.h"
#include "kata_records.h"

#include <algorithm>

namespace kata {

namespace {

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// a * x + y, elementwise (the decayed combine; a = 1 is plain addition)
__device__ __forceinline__ float4 axpy4(float a, float4 x, float4 y) {
    return make_float4(__builtin_fmaf(a, x.x, y.x), __builtin_fmaf(a, x.y, y.y),
                       __builtin_fmaf(a, x.z, y.z), __builtin_fmaf(a, x.w, y.w));
}

// The four total elements 4 e4 .. 4 e4 + 3 of sequence seq, written to the
// packed state in place of a separate conversion pass.
__device__ __forceinline__ void export_total(const RecordExport& ex, size_t seq, int e4, float4 t) {
    export_element(ex, seq, 4 * e4 + 0, t.x);
    export_element(ex, seq, 4 * e4 + 1, t.y);
    export_element(ex, seq, 4 * e4 + 2, t.z);
    export_element(ex, seq, 4 * e4 + 3, t.w);
}

// Few records per sequence (NR <= kSeqMax): one thread per 4 consecutive
// elements walks the records in order. Loads are issued 8 records ahead of the
// dependent adds, so every thread keeps 8 coalesced 16-byte reads in flight.
constexpr int kSeqMax = 32;
constexpr int kSeqUnroll = 8;

template <bool DECAY>
__global__ __launch_bounds__(256) void scan_records_seq_kernel(
    float* __restrict__ rec, const float* __restrict__ dec, int NR, int E,
    const float* __restrict__ init, float* __restrict__ total_a, float* __restrict__ total_b,
    RecordExport ex) {
    const size_t seq = blockIdx.y;
    const int E4 = E / 4;
    const int e4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (e4 >= E4) return;
    float4* base = reinterpret_cast<float4*>(rec + seq * (size_t)NR * E) + e4;
    float4 carry = init ? reinterpret_cast<const float4*>(init + seq * E)[e4]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r0 = 0; r0 < NR; r0 += kSeqUnroll) {
        float4 x[kSeqUnroll];
#pragma unroll
        for (int i = 0; i < kSeqUnroll; ++i)
            if (r0 + i < NR) x[i] = base[(size_t)(r0 + i) * E4];
#pragma unroll
        for (int i = 0; i < kSeqUnroll; ++i)
            if (r0 + i < NR) {
                base[(size_t)(r0 + i) * E4] = carry;
                carry = DECAY ? axpy4(dec[seq * NR + r0 + i], carry, x[i]) : add4(carry, x[i]);
            }
    }
    if (total_a) reinterpret_cast<float4*>(total_a + seq * E)[e4] = carry;
    if (total_b) reinterpret_cast<float4*>(total_b + seq * E)[e4] = carry;
    if (ex.layout != kRecNone) export_total(ex, seq, e4, carry);
}

// Blocked two-level scan. A block owns kCols4 float4 columns of one sequence
// and walks its records in tiles of kGroups * kPer: thread (group g, column c)
// holds records g*kPer .. g*kPer + kPer - 1 of the tile in registers, sums them,
// publishes the sum in LDS, takes the sum of the groups before it (plus the
// running carry of earlier tiles) as its offset, and writes its records'
// exclusive prefixes.
constexpr int kCols4 = 32;
constexpr int kGroups = 8;
constexpr int kPer = 16;
constexpr int kTileRecs = kGroups * kPer;

template <bool DECAY>
__global__ __launch_bounds__(kCols4 * kGroups) void scan_records_blocked_kernel(
    float* __restrict__ rec, const float* __restrict__ dec, int NR, int E,
    const float* __restrict__ init, float* __restrict__ total_a, float* __restrict__ total_b,
    RecordExport ex) {
    __shared__ float4 gsum[kGroups][kCols4];
    __shared__ float gdec[kGroups];
    const size_t seq = blockIdx.y;
    const int E4 = E / 4;
    const int c = threadIdx.x % kCols4, g = threadIdx.x / kCols4;
    const int e4 = blockIdx.x * kCols4 + c;
    const bool col_ok = e4 < E4;
    // loads always read a valid address (clamped column and record) and the
    // value is zeroed afterwards, so no pointer select reaches the load
    float4* base = reinterpret_cast<float4*>(rec + seq * (size_t)NR * E) + e4;
    const float4* load_base =
        reinterpret_cast<const float4*>(rec + seq * (size_t)NR * E) + min(e4, E4 - 1);
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 carry = zero;
    if (init) {
        const float4 i4 = reinterpret_cast<const float4*>(init + seq * E)[min(e4, E4 - 1)];
        if (col_ok) carry = i4;
    }
    for (int r0 = 0; r0 < NR; r0 += kTileRecs) {
        const int rg = r0 + g * kPer;
        float4 x[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const float4 t = load_base[(size_t)min(rg + i, NR - 1) * E4];
            const bool ok = col_ok && rg + i < NR;
            x[i] = make_float4(ok ? t.x : 0.f, ok ? t.y : 0.f, ok ? t.z : 0.f, ok ? t.w : 0.f);
        }
        // decays of this thread's records; records past the end are the
        // identity (a = 1, S = 0)
        float a[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) a[i] = DECAY && rg + i < NR ? dec[seq * NR + rg + i] : 1.0f;
        float4 s = zero;
        float ag = 1.0f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            s = DECAY ? axpy4(a[i], s, x[i]) : add4(s, x[i]);
            ag *= a[i];
        }
        gsum[g][c] = s;
        if (DECAY && c == 0) gdec[g] = ag;
        __syncthreads();
        float4 off = carry, tot = carry;
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const float4 gj = gsum[j][c];
            if (DECAY) {
                const float aj = gdec[j];
                if (j < g) off = axpy4(aj, off, gj);
                tot = axpy4(aj, tot, gj);
            } else {
                if (j < g) off = add4(off, gj);
                tot = add4(tot, gj);
            }
        }
        __syncthreads();                           // gsum is rewritten by the next tile
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (col_ok && rg + i < NR) base[(size_t)(rg + i) * E4] = off;
            off = DECAY ? axpy4(a[i], off, x[i]) : add4(off, x[i]);
        }
        carry = tot;
    }
    if (g == 0 && col_ok) {
        if (total_a) reinterpret_cast<float4*>(total_a + seq * E)[e4] = carry;
        if (total_b) reinterpret_cast<float4*>(total_b + seq * E)[e4] = carry;
        if (ex.layout != kRecNone) export_total(ex, seq, e4, carry);
    }
}

// ---- log-depth (tree) variant -------------------------------------------------
// Reduce-then-scan over tiles of kTreeTile records. Within a tile the records
// of kTreeCols float4 columns sit in LDS and a Kogge-Stone scan combines
// element r with element r - 2^k for k = 0 .. log2(tile) - 1 (every level one
// dependent combine; with the gate, element r carries its span's decay A_r and
// the combine of (A1, S1) before (A2, S2) is (A1 A2, A2 S1 + S2)). Each tile
// writes its records' tile-local exclusive prefixes in place and its total to
// the tile-sums array; the tile sums are scanned by the same scheme (one level
// up) and a last pass combines every record with its tile's offset. Depth:
// ceil(log2 n) levels per tile pass plus one combine per level of tiles.
constexpr int kTreeTile = 128;
constexpr int kTreeCols = 8;
constexpr int kTreeThreads = 256;
constexpr int kTreePer = kTreeTile * kTreeCols / kTreeThreads;   // elements per thread

__device__ __forceinline__ float4 scale4(float a, float4 x) {
    return make_float4(a * x.x, a * x.y, a * x.z, a * x.w);
}

// One tile (blockIdx.z) of kTreeCols columns (blockIdx.x) of sequence
// blockIdx.y. init (NULL = 0) is folded in when the sequence is one tile;
// tsum / tdec (NULL when one tile) receive the tile's total and decay, and
// rdec each record's tile-local exclusive decay (the gated apply pass uses it).
template <bool DECAY>
__global__ __launch_bounds__(kTreeThreads) void scan_tree_tile_kernel(
    float* __restrict__ rec, const float* __restrict__ dec, int NR, int E,
    const float* __restrict__ init, float* __restrict__ tsum, float* __restrict__ tdec,
    float* __restrict__ rdec, float* __restrict__ total_a, float* __restrict__ total_b,
    RecordExport ex) {
    __shared__ float4 buf[2][kTreeTile][kTreeCols];
    __shared__ float abuf[2][kTreeTile];
    const size_t seq = blockIdx.y;
    const int NT = (NR + kTreeTile - 1) / kTreeTile, tile = blockIdx.z;
    const int E4 = E / 4;
    const int c = threadIdx.x % kTreeCols, rb = threadIdx.x / kTreeCols;   // rows rb + 32 i
    const int e4 = blockIdx.x * kTreeCols + c;
    const bool col_ok = e4 < E4;
    const int r0 = tile * kTreeTile, n = min(kTreeTile, NR - r0);
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4* base = reinterpret_cast<float4*>(rec + (seq * (size_t)NR + r0) * E) + e4;
    const float4* load_base =
        reinterpret_cast<const float4*>(rec + (seq * (size_t)NR + r0) * E) + min(e4, E4 - 1);
#pragma unroll
    for (int i = 0; i < kTreePer; ++i) {
        const int r = rb + (kTreeThreads / kTreeCols) * i;
        const float4 t = load_base[(size_t)min(r, n - 1) * E4];
        const bool ok = col_ok && r < n;
        buf[0][r][c] = make_float4(ok ? t.x : 0.f, ok ? t.y : 0.f, ok ? t.z : 0.f, ok ? t.w : 0.f);
    }
    if (DECAY && threadIdx.x < kTreeTile)
        abuf[0][threadIdx.x] = threadIdx.x < n ? dec[seq * NR + r0 + threadIdx.x] : 1.0f;
    __syncthreads();
    int cur = 0;
    for (int d = 1; d < n; d <<= 1) {                 // Kogge-Stone: one level per d
#pragma unroll
        for (int i = 0; i < kTreePer; ++i) {
            const int r = rb + (kTreeThreads / kTreeCols) * i;
            float4 x = buf[cur][r][c];
            if (r >= d) {
                const float4 y = buf[cur][r - d][c];
                x = DECAY ? axpy4(abuf[cur][r], y, x) : add4(y, x);
            }
            buf[cur ^ 1][r][c] = x;
        }
        if (DECAY && threadIdx.x < kTreeTile) {
            const int r = threadIdx.x;
            abuf[cur ^ 1][r] = r >= d ? abuf[cur][r - d] * abuf[cur][r] : abuf[cur][r];
        }
        __syncthreads();
        cur ^= 1;
    }
    // exclusive prefix of record r: inclusive value of r - 1 (init folded in
    // when the sequence is a single tile; its decay to r is the inclusive A of r - 1)
    const bool single = NT == 1;
    float4 i4 = zero;
    if (single && init && col_ok) i4 = reinterpret_cast<const float4*>(init + seq * E)[e4];
#pragma unroll
    for (int i = 0; i < kTreePer; ++i) {
        const int r = rb + (kTreeThreads / kTreeCols) * i;
        if (col_ok && r < n) {
            float4 p = r > 0 ? buf[cur][r - 1][c] : zero;
            if (single) p = DECAY ? axpy4(r > 0 ? abuf[cur][r - 1] : 1.0f, i4, p) : add4(i4, p);
            base[(size_t)r * E4] = p;
        }
    }
    if (rb == 0 && col_ok) {
        float4 t = buf[cur][n - 1][c];
        if (single) {
            t = DECAY ? axpy4(abuf[cur][n - 1], i4, t) : add4(i4, t);
            if (total_a) reinterpret_cast<float4*>(total_a + seq * E)[e4] = t;
            if (total_b) reinterpret_cast<float4*>(total_b + seq * E)[e4] = t;
            if (ex.layout != kRecNone) export_total(ex, seq, e4, t);
        } else {
            reinterpret_cast<float4*>(tsum + (seq * (size_t)NT + tile) * E)[e4] = t;
        }
    }
    if (DECAY && !single && blockIdx.x == 0) {
        if (threadIdx.x == 0) tdec[seq * NT + tile] = abuf[cur][n - 1];
        if (threadIdx.x < n) rdec[seq * NR + r0 + threadIdx.x] = threadIdx.x > 0 ? abuf[cur][threadIdx.x - 1] : 1.0f;
    }
}

// Combines every record of tile t with the tile's exclusive offset (the scanned
// tile sums): with the gate, offset decayed by the record's tile-local
// exclusive decay rdec (the product of the decays of the tile's records before
// it, from the tile pass).
template <bool DECAY>
__global__ __launch_bounds__(kTreeThreads) void scan_tree_apply_kernel(
    float* __restrict__ rec, const float* __restrict__ rdec, int NR, int E,
    const float* __restrict__ toff) {
    const size_t seq = blockIdx.y;
    const int NT = (NR + kTreeTile - 1) / kTreeTile, tile = blockIdx.z;
    const int E4 = E / 4;
    const int c = threadIdx.x % kTreeCols, rb = threadIdx.x / kTreeCols;
    const int e4 = blockIdx.x * kTreeCols + c;
    if (e4 >= E4) return;
    const int r0 = tile * kTreeTile, n = min(kTreeTile, NR - r0);
    const float4 off = reinterpret_cast<const float4*>(toff + (seq * (size_t)NT + tile) * E)[e4];
    float4* base = reinterpret_cast<float4*>(rec + (seq * (size_t)NR + r0) * E) + e4;
    for (int r = rb; r < n; r += kTreeThreads / kTreeCols) {
        float4 p = base[(size_t)r * E4];
        if (DECAY) {
            p = axpy4(rdec[seq * NR + r0 + r], off, p);
        } else {
            p = add4(off, p);
        }
        base[(size_t)r * E4] = p;
    }
}

// Levels of dependent combines the tree scan takes over n records.
int tree_levels(int n) {
    if (n <= 1) return n;                                  // the init combine only
    int lg = 0;
    while ((1 << lg) < std::min(n, kTreeTile)) ++lg;
    if (n <= kTreeTile) return lg + 1;                     // tile scan, then the init
    return lg + tree_levels((n + kTreeTile - 1) / kTreeTile) + 1;   // tiles, offsets, apply
}

template <bool DECAY>
hipError_t scan_tree_impl(float* rec, const float* dec, int nseq, int NR, int E,
                          const float* init, float* total_a, float* total_b, float* scratch,
                          hipStream_t st, const RecordExport& x) {
    if (NR == 0) return hipSuccess;
    const int NT = (NR + kTreeTile - 1) / kTreeTile;
    dim3 grid((E / 4 + kTreeCols - 1) / kTreeCols, nseq, NT);
    // this level's scratch: tile sums [nseq, NT, E], then (gated) tile decays
    // [nseq, NT] and record decays [nseq, NR]
    float* tsum = NT > 1 ? scratch : nullptr;
    float* tdec = NT > 1 && DECAY ? scratch + (size_t)nseq * NT * E : nullptr;
    float* rdec = NT > 1 && DECAY ? tdec + (size_t)nseq * NT : nullptr;
    scan_tree_tile_kernel<DECAY><<<grid, kTreeThreads, 0, st>>>(rec, dec, NR, E, init, tsum, tdec,
                                                                rdec, total_a, total_b, x);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || NT == 1) return e;
    // tile sums -> exclusive tile offsets (and the totals), one level up
    float* next = scratch + (size_t)nseq * NT * E + (DECAY ? (size_t)nseq * (NT + NR) : 0);
    e = scan_tree_impl<DECAY>(tsum, tdec, nseq, NT, E, init, total_a, total_b, next, st, x);
    if (e != hipSuccess) return e;
    scan_tree_apply_kernel<DECAY><<<grid, kTreeThreads, 0, st>>>(rec, rdec, NR, E, tsum);
    return hipGetLastError();
}

__global__ void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                    size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.0f;
}

template <bool DECAY>
hipError_t scan_impl(float* rec, const float* dec, int nseq, int NR, int E, const float* init,
                     float* total_a, float* total_b, hipStream_t st, const RecordExport* ex) {
    if (nseq == 0 || E == 0) return hipSuccess;
    if (E % 4 != 0) return hipErrorInvalidValue;      // every record length is a multiple of 4
    const RecordExport x = ex ? *ex : RecordExport{kRecNone, 0, 0, nullptr, nullptr};
    if (NR <= kSeqMax) {
        dim3 grid((E / 4 + 255) / 256, nseq);
        scan_records_seq_kernel<DECAY><<<grid, 256, 0, st>>>(rec, dec, NR, E, init, total_a, total_b,
                                                             x);
    } else {
        dim3 grid((E / 4 + kCols4 - 1) / kCols4, nseq);
        scan_records_blocked_kernel<DECAY><<<grid, kCols4 * kGroups, 0, st>>>(rec, dec, NR, E, init,
                                                                              total_a, total_b, x);
    }
    return hipGetLastError();
}

}  // namespace

size_t scan_tree_scratch_floats(int nseq, int NR, int E, bool decay) {
    size_t n = 0;
    while (NR > kTreeTile) {
        const int NT = (NR + kTreeTile - 1) / kTreeTile;
        n += (size_t)nseq * NT * E + (decay ? (size_t)nseq * (NT + NR) : 0);
        NR = NT;
    }
    return n;
}

int scan_levels(int NR, int method) {
    if (NR <= 0) return 0;
    if (method == 1) return NR;                            // sequential walk
    if (method == 2) return tree_levels(NR);               // tree
    if (NR <= kSeqMax) return NR;                          // blocked scan: per-element walk
    // per thread kPer records, the group offsets, the carry across tiles
    return kPer + kGroups + (NR + kTileRecs - 1) / kTileRecs;
}

hipError_t launch_scan_records_tree(float* rec, const float* dec, int nseq, int NR, int E,
                                    const float* init, float* total_a, float* total_b,
                                    float* scratch, hipStream_t st, const RecordExport* ex) {
    if (nseq == 0 || E == 0) return hipSuccess;
    if (E % 4 != 0) return hipErrorInvalidValue;
    // the depth the pages give the associative scan: O(log n); checked here as
    // ceil(log2 n) plus two combines per level of tiles
    int lg = 0, tl = 0;
    while ((1 << lg) < NR) ++lg;
    for (int n = NR; n > 1; n = (n + kTreeTile - 1) / kTreeTile) ++tl;
    if (tree_levels(NR) > lg + 2 * std::max(tl, 1)) return hipErrorInvalidValue;
    const RecordExport x = ex ? *ex : RecordExport{kRecNone, 0, 0, nullptr, nullptr};
    return dec ? scan_tree_impl<true>(rec, dec, nseq, NR, E, init, total_a, total_b, scratch, st, x)
               : scan_tree_impl<false>(rec, nullptr, nseq, NR, E, init, total_a, total_b, scratch,
                                       st, x);
}

hipError_t launch_scan_records(float* rec, int nseq, int NR, int E, const float* init,
                               float* total_a, float* total_b, hipStream_t st,
                               const RecordExport* ex) {
    return scan_impl<false>(rec, nullptr, nseq, NR, E, init, total_a, total_b, st, ex);
}

hipError_t launch_scan_records_decay(float* rec, const float* dec, int nseq, int NR, int E,
                                     const float* init, float* total_a, float* total_b,
                                     hipStream_t st, const RecordExport* ex) {
    return scan_impl<true>(rec, dec, nseq, NR, E, init, total_a, total_b, st, ex);
}

hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    copy_or_zero_kernel<<<(unsigned)blocks, 256, 0, st>>>(dst, src, n);
    return hipGetLastError();
}

}  // namespace kata
