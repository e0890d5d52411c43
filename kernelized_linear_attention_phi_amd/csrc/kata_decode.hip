// Recurrent decode step: S += phi(k) v^T, z += phi(k), o = phi(q).S / phi(q).z.
//
// The constant-time recurrent inference with a fixed-size state that the KATA
// abstract (arXiv 2607.17419) and the linear-attention definition (notes.yuuk.io,
// "Definition": an exact RNN with a fixed-dimension state) describe; the read
// follows the update, so the token attends to itself (the output gate of the
// KATA explainers, section 2.1, blends the previous readout with the current
// value).
//
// HBM-bound: per (sequence, head) the fp32 state (D*dv + D floats) is read once
// and written once. One block per row; every thread owns DV/4-float columns of
// a fixed set of state rows, loads all of them before any store (so the loads
// are in flight together), updates, stores with 16-byte accesses, and keeps a
// partial phi(q).S; partials are reduced through LDS.
//
// Decay-gated variant: with a per-row log-decay g <= 0 the update is
// S = exp(g) S + phi(k) v^T, z = exp(g) z + phi(k) (the state decays before the
// token is added), the same read follows.
#include "kata_device.h"
#include "kata_internal.h"

namespace kata {

namespace {

constexpr int kThreads = 256;

template <typename TIn, int DK, int DV, bool DECAY>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ gdec, float* __restrict__ S, float* __restrict__ z,
    TIn* __restrict__ o) {
    constexpr int D = DK * (DK + 1) / 2;
    constexpr int C4 = DV / 4;              // float4 columns per row
    constexpr int RG = kThreads / C4;       // row groups
    constexpr int RPT = (D + RG - 1) / RG;  // rows per thread
    __shared__ float fq[D], fk[D], vs[DV], qs[DK], ks[DK];
    __shared__ float4 red[RG][C4];
    __shared__ float dred[kThreads / 64];

    const size_t row = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < DK) {
        qs[tid] = io<TIn>::ld(q, row * DK + tid);
        ks[tid] = io<TIn>::ld(k, row * DK + tid);
    }
    if (tid < DV) vs[tid] = io<TIn>::ld(v, row * DV + tid);
    __syncthreads();
    for (int p = tid; p < D; p += kThreads) {
        const uint32_t pr = pack_pair(p, DK);
        const int i = pr & 0xff, j = pr >> 8;
        const float sc = i == j ? 1.0f : kSqrt2;
        fq[p] = sc * (qs[i] * qs[j]);
        fk[p] = sc * (ks[i] * ks[j]);
    }
    __syncthreads();

    const int rg = tid / C4, c4 = tid % C4;
    float4* S4 = reinterpret_cast<float4*>(S + row * (size_t)D * DV);
    float4 cur[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int p = rg + u * RG;
        if (p < D) cur[u] = S4[p * C4 + c4];
    }
    const float4 vv = reinterpret_cast<const float4*>(vs)[c4];
    const float gam = DECAY ? expf(gdec[row]) : 1.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int p = rg + u * RG;
        if (p < D) {
            const float a = fk[p], b = fq[p];
            float4 s = cur[u];
            if (DECAY) {
                s.x = __builtin_fmaf(gam, s.x, a * vv.x);
                s.y = __builtin_fmaf(gam, s.y, a * vv.y);
                s.z = __builtin_fmaf(gam, s.z, a * vv.z);
                s.w = __builtin_fmaf(gam, s.w, a * vv.w);
            } else {
                s.x += a * vv.x; s.y += a * vv.y; s.z += a * vv.z; s.w += a * vv.w;
            }
            S4[p * C4 + c4] = s;
            acc.x += b * s.x; acc.y += b * s.y; acc.z += b * s.z; acc.w += b * s.w;
        }
    }
    red[rg][c4] = acc;

    float dpart = 0.0f;
    float* zr = z + row * (size_t)D;
    for (int p = tid; p < D; p += kThreads) {
        const float zn = DECAY ? __builtin_fmaf(gam, zr[p], fk[p]) : zr[p] + fk[p];
        zr[p] = zn;
        dpart += fq[p] * zn;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off, 64);
    if ((tid & 63) == 0) dred[tid >> 6] = dpart;
    __syncthreads();

    if (tid < DV) {
        const int cc = tid / 4, w = tid % 4;
        float num = 0.0f;
        for (int g = 0; g < RG; ++g) {
            const float4 r = red[g][cc];
            num += w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
        }
        float den = 0.0f;
#pragma unroll
        for (int u = 0; u < kThreads / 64; ++u) den += dred[u];
        io<TIn>::st(o, row * DV + tid, safe_div(num, den));
    }
}

template <typename TIn, int DK, int DV>
void launch_dk_dv(const TIn* q, const TIn* k, const TIn* v, const float* g, float* S, float* z,
                  TIn* o, int N, hipStream_t st) {
    if (g) decode_kernel<TIn, DK, DV, true><<<N, kThreads, 0, st>>>(q, k, v, g, S, z, o);
    else decode_kernel<TIn, DK, DV, false><<<N, kThreads, 0, st>>>(q, k, v, nullptr, S, z, o);
}

template <typename TIn, int DK>
hipError_t launch_dk(const void* q, const void* k, const void* v, const float* g, float* S,
                     float* z, void* o, int N, int dv, hipStream_t st) {
    const TIn* qq = (const TIn*)q;
    const TIn* kk = (const TIn*)k;
    const TIn* vv = (const TIn*)v;
    TIn* oo = (TIn*)o;
    switch (dv) {
        case 16: launch_dk_dv<TIn, DK, 16>(qq, kk, vv, g, S, z, oo, N, st); break;
        case 32: launch_dk_dv<TIn, DK, 32>(qq, kk, vv, g, S, z, oo, N, st); break;
        case 64: launch_dk_dv<TIn, DK, 64>(qq, kk, vv, g, S, z, oo, N, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* g, float* S,
                    float* z, void* o, int N, int dk, int dv, hipStream_t st) {
    if (dk == 16) return launch_dk<TIn, 16>(q, k, v, g, S, z, o, N, dv, st);
    if (dk == 32) return launch_dk<TIn, 32>(q, k, v, g, S, z, o, N, dv, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g, float* S,
                         float* z, void* o, int N, int dk, int dv, bool bf16, hipStream_t st) {
    if (N == 0) return hipSuccess;
    return bf16 ? launch_t<bf16_t>(q, k, v, g, S, z, o, N, dk, dv, st)
                : launch_t<float>(q, k, v, g, S, z, o, N, dk, dv, st);
}

}  // namespace kata
