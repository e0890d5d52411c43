// State-record layouts of the matrix-core kernels and their map to the packed
// state the boundary exchanges (S [D, d_v] with the packed feature order
// p(i, j) = i d - i(i - 1)/2 + (j - i), z [D]). A record holds one state in
// accumulator order; the packed state holds sqrt(2) x_i x_j features where the
// records hold x_i x_j (the factor sits on the query side inside the kernels).
#pragma once

#include "kata_device.h"
#include "kata_internal.h"

namespace kata {

// d_k = 16 record (nine feature tiles delta = 0..8 of 16 rows rho: x_rho x_{rho+delta},
// tile 8 rows rho >= 8 unused; then the Gram matrix): element idx -> packed
// index (-1: no packed counterpart), value column (-1: z), scale, and whether it
// is a lower-triangle Gram entry (skipped on export, filled on import).
__device__ __forceinline__ int rec16_to_packed(int idx, int NTV, int* col, float* scale,
                                               bool* lower) {
    constexpr int DK = 16, NMT = 9;
    const int sz = NMT * NTV * 256;
    *lower = false;
    if (idx >= sz) {                                 // Gram matrix Z[i][j]
        const int e = idx - sz;
        const int lane = (e >> 2) & 63;
        const int i = 4 * (lane >> 4) + (e & 3), j = lane & 15;
        const int a = min(i, j), b = max(i, j);
        *col = -1;
        *scale = i == j ? 1.0f : kSqrt2;
        *lower = i > j;
        return a * DK - a * (a - 1) / 2 + (b - a);
    }
    const int r = idx & 3, lane = (idx >> 2) & 63, nt = (idx >> 8) % NTV;
    const int d = (idx >> 8) / NTV;
    const int rho = 4 * (lane >> 4) + r;
    *col = 16 * nt + (lane & 15);
    if (d == 8 && rho >= 8) return -1;
    const int i = rho, j = (rho + d) & 15;
    const int a = min(i, j), b = max(i, j);
    *scale = d == 0 ? 1.0f : kSqrt2;
    return a * DK - a * (a - 1) / 2 + (b - a);
}

// d_k = 32 record (33 feature tiles: L-circulant, U-circulant, cross, mixed;
// then four Gram tiles LL, LU, UL, UU): as above.
__device__ __forceinline__ int rec32_to_packed(int idx, int NTV, int* col, float* scale,
                                               bool* lower) {
    constexpr int DK = 32, NFT = 33;
    const int sz = NFT * NTV * 256;
    int a, b;
    *lower = false;
    if (idx >= sz) {                                 // Gram tile zt, Z[i][j]
        const int e = idx - sz;
        const int zt = e >> 8, lane = (e >> 2) & 63;
        const int i = 4 * (lane >> 4) + (e & 3), j = lane & 15;
        a = i + ((zt >> 1) ? 16 : 0);                // row half: L for LL, LU; U for UL, UU
        b = j + ((zt & 1) ? 16 : 0);                 // column half: L for LL, UL; U for LU, UU
        *col = -1;
        *lower = a > b;
    } else {
        const int r = idx & 3, lane = (idx >> 2) & 63, nt = (idx >> 8) % NTV;
        const int t = (idx >> 8) / NTV;
        const int rho = 4 * (lane >> 4) + r;
        *col = 16 * nt + (lane & 15);
        if (t < 8) { a = rho; b = (rho + t) & 15; }
        else if (t < 16) { a = 16 + rho; b = 16 + ((rho + t - 8) & 15); }
        else if (t < 32) { a = rho; b = 16 + ((rho + t - 16) & 15); }
        else if (rho < 8) { a = rho; b = rho + 8; }
        else { a = 8 + rho; b = 16 + rho; }
    }
    *scale = a == b ? 1.0f : kSqrt2;
    const int i = min(a, b), j = max(a, b);
    return i * DK - i * (i - 1) / 2 + (j - i);
}

// First-order and factored-feature record (units (at, u) of 256 floats, u = NTV
// the z tile whose column 0 holds z): element e -> feature a, value column, and
// whether it is in the z tile. The last feature tile may run past the feature
// count (its rows stay zero).
__device__ __forceinline__ void rec1_coords(int e, int NTV, int* a, int* col, bool* zt) {
    const int unit = e / 256, lane = (e % 256) / 4, r = e % 4;
    const int at = unit / (NTV + 1), u = unit % (NTV + 1);
    *a = 16 * at + 4 * (lane / 16) + r;
    *zt = u == NTV;
    *col = *zt ? lane % 16 : 16 * u + lane % 16;
}

// Writes element idx (value val) of sequence b's record to the packed state.
__device__ __forceinline__ void export_element(const RecordExport& x, size_t b, int idx, float val) {
    const int NTV = x.dv / 16;
    if (x.layout == kRecIdent) {
        int a, col;
        bool zt;
        rec1_coords(idx, NTV, &a, &col, &zt);
        if (a >= x.dk) return;                     // rows past the feature count
        if (!zt) x.S[(b * x.dk + a) * x.dv + col] = val;
        else if (col == 0) x.z[b * x.dk + a] = val;
        return;
    }
    int col;
    float scale;
    bool lower;
    const int p = x.layout == kRecPsd16 ? rec16_to_packed(idx, NTV, &col, &scale, &lower)
                                        : rec32_to_packed(idx, NTV, &col, &scale, &lower);
    if (p < 0 || lower) return;
    const size_t D = (size_t)x.dk * (x.dk + 1) / 2;
    if (col >= 0) x.S[(b * D + p) * x.dv + col] = val * scale;
    else x.z[b * D + p] = val * scale;
}

}  // namespace kata
