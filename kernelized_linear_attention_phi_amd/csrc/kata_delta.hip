// DeltaKATA: the delta rule on the KATA state (gfx950, fp32 arithmetic).
//
// The KATA explainers (gist.science, technical summary 4) name a delta-rule
// variant that corrects stale bindings at repeated keys; the reading built here
// applies the delta rule of DeltaNet (summary 1) to the augmented state
// A = [S | z] with the unit-norm lifted key kappa_t = phi(k_t) / |k_t|^2, a write
// strength beta_t and the value u_t = [v_t, 1]:
//     A_t = A_{t-1} + beta_t kappa_t (u_t - kappa_t^T A_{t-1}),
//     o_t = phi(q_t).S_t / phi(q_t).z_t            (0 where the denominator is 0).
// The state update is matrix-affine, so chunks are walked in order (the
// explainers' chunked-state form, summary 2.3, with the delta rule's chunk
// recursion): inside chunk c with the state A before it,
//     R = U - K A                      (K rows kappa_t),
//     (I + diag(beta) L) P = diag(beta) R,   L the strictly lower part of K K^T,
//     O = phi(Q) A + mask(phi(Q) K^T) P      (inclusive causal mask),
//     A <- A + K^T P.
// The triangular system is solved in blocks of 16 rows: the inverse of each
// unit lower-triangular 16 x 16 diagonal block by forward substitution (one
// thread per column), then block rows in order, each a product with the
// earlier blocks' P and with its block inverse.
//
// One workgroup of 16 wavefronts per (batch, head, 16-column value tile) keeps
// its 16 columns of S and the z column in LDS (the z column is recomputed by
// every value tile of a head); the products R, O and K^T P are spread one
// (token, column) or (feature, column) per thread. At d_k = 16 the chunk's
// lifted keys and queries are formed once per chunk in LDS; at d_k = 32 (528
// features, too many to hold beside the state) on the fly through a pair
// table. Everything is fp32.
#include "kata_device.h"
#include "kata_internal.h"
#include "kata_mfma.h"

namespace kata {

namespace {

constexpr int kThreads = 256;          // decode
constexpr int kFwdThreads = 1024;      // forward: 16 wavefronts per (head, value tile)
constexpr int kCols = 17;              // 16 value columns + z
constexpr int kSub = 16;               // rows per block of the triangular solve

template <int DK, int C>
struct DeltaCfg {
    static constexpr int D = DK * (DK + 1) / 2;
    static constexpr int NB = C / kSub;
    // LDS layout, in floats
    static constexpr int S_OFF = 0;                           // state [D][17]
    static constexpr int K_OFF = S_OFF + D * kCols;           // keys [C][DK]
    static constexpr int Q_OFF = K_OFF + C * DK;              // queries [C][DK]
    static constexpr int U_OFF = Q_OFF + C * DK;              // [v | 1] [C][17]
    static constexpr int INV_OFF = U_OFF + C * kCols;         // 1 / |k_t|^2 [C]
    static constexpr int B_OFF = INV_OFF + C;                 // beta [C]
    static constexpr int G_OFF = B_OFF + C;                   // beta_t kappa_t.kappa_j, j < t [C][C]
    static constexpr int A_OFF = G_OFF + C * C;               // phi(q_t).kappa_j, j <= t [C][C]
    static constexpr int R_OFF = A_OFF + C * C;               // R, then the block right-hand sides [C][17]
    static constexpr int P_OFF = R_OFF + C * kCols;           // P [C][17]
    static constexpr int TI_OFF = P_OFF + C * kCols;          // block inverses [NB][16][16]
    static constexpr int O_OFF = TI_OFF + NB * kSub * kSub;   // outputs [C][17]
    static constexpr int BASE = O_OFF + C * kCols;
    // the chunk's lifted keys kappa [C][D] and queries phi(q) [C][D], formed
    // once per chunk where they fit next to the rest (d_k = 16)
    static constexpr bool PRE = (BASE + 2 * C * D) * 4 + D * 4 <= 150 * 1024;
    static constexpr int KAP_OFF = BASE;
    static constexpr int FQ_OFF = KAP_OFF + C * D;
    static constexpr int FLOATS = PRE ? FQ_OFF + C * D : BASE;
    static_assert(C % kSub == 0 && NB * kSub <= kFwdThreads && kSub * kCols <= kFwdThreads,
                  "chunk of 16, 32 or 64");
    static_assert(FLOATS * 4 + D * 4 <= 160 * 1024, "fits the LDS of a compute unit");
};

// D = A(16x4) * B(4x16) + C in fp32 (v_mfma_f32_16x16x4_f32): fp32 operands,
// fp32 accumulation.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TIn, int DK, int C>
__global__ __launch_bounds__(kFwdThreads) void delta_fwd_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ beta, TIn* __restrict__ o, const float* __restrict__ S0,
    const float* __restrict__ z0, float* __restrict__ S_out, float* __restrict__ z_out, int T,
    int DV) {
    using F = DeltaCfg<DK, C>;
    constexpr int D = F::D, NT = kFwdThreads;
    __shared__ float sm[F::FLOATS];
    __shared__ uint32_t pairs[D];
    float* St = sm + F::S_OFF;
    float* Ks = sm + F::K_OFF;
    float* Qs = sm + F::Q_OFF;
    float* Us = sm + F::U_OFF;
    float* Inv = sm + F::INV_OFF;
    float* Bs = sm + F::B_OFF;
    float* G = sm + F::G_OFF;
    float* Aq = sm + F::A_OFF;
    float* R = sm + F::R_OFF;
    float* P = sm + F::P_OFF;
    float* TI = sm + F::TI_OFF;
    float* Os = sm + F::O_OFF;
    float* Kap = sm + F::KAP_OFF;              // PRE only
    float* Fq = sm + F::FQ_OFF;                // PRE only

    const int vt = blockIdx.x;                 // value tile: columns 16 vt .. 16 vt + 15
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;

    for (int p = tid; p < D; p += NT) pairs[p] = pack_pair(p, DK);
    for (int e = tid; e < D * kCols; e += NT) {
        const int p = e / kCols, c = e % kCols;
        float x = 0.0f;
        if (S0) x = c < kSub ? S0[(bh * D + p) * DV + kSub * vt + c] : z0[bh * D + p];
        St[e] = x;
    }
    __syncthreads();

    // lifted key (kappa, scaled by 1 / |k_t|^2) and query of token t, feature p
    auto kappa = [&](int t, int p) -> float {
        if constexpr (F::PRE) {
            return Kap[t * D + p];
        } else {
            const uint32_t pr = pairs[p];
            const int a = pr & 0xff, b = pr >> 8;
            return Ks[t * DK + a] * Ks[t * DK + b] * ((a == b ? 1.0f : kSqrt2) * Inv[t]);
        }
    };
    auto phiq = [&](int t, int p) -> float {
        if constexpr (F::PRE) {
            return Fq[t * D + p];
        } else {
            const uint32_t pr = pairs[p];
            const int a = pr & 0xff, b = pr >> 8;
            return Qs[t * DK + a] * Qs[t * DK + b] * (a == b ? 1.0f : kSqrt2);
        }
    };

    // matrix-core tiles: wavefront w takes tiles w, w + 16, ...; lane (c16, g)
    // of a 16x16x4 fp32 product holds A[row c16][k g], B[k g][column c16] and
    // accumulator rows 4g + r of column c16
    const int wave = tid >> 6, lane = tid & 63, c16 = lane & 15, g4 = lane >> 4;
    constexpr int NWV = NT / 64;
    constexpr int MT = C / 16;                      // token tiles
    constexpr int FT = (D + 15) / 16;               // feature tiles

    for (int c0 = 0; c0 < T; c0 += C) {
        const int n = min(C, T - c0);
        const size_t tok0 = bh * (size_t)T + c0;
        // ---- stage the chunk (rows past a ragged end are zero: no key, no
        // write, beta 0)
        for (int e = tid; e < C * DK; e += NT) {
            const int t = e / DK;
            Ks[e] = t < n ? io<TIn>::ld(k, tok0 * DK + e) : 0.0f;
            Qs[e] = t < n ? io<TIn>::ld(q, tok0 * DK + e) : 0.0f;
        }
        for (int e = tid; e < C * kCols; e += NT) {
            const int t = e / kCols, c = e % kCols;
            float x = 0.0f;
            if (t < n) x = c < kSub ? io<TIn>::ld(v, (tok0 + t) * DV + kSub * vt + c) : 1.0f;
            Us[e] = x;
        }
        for (int t = tid; t < C; t += NT) Bs[t] = t < n ? beta[tok0 + t] : 0.0f;
        __syncthreads();
        for (int t = tid; t < C; t += NT) {
            float s = 0.0f;
#pragma unroll
            for (int a = 0; a < DK; ++a) s = __builtin_fmaf(Ks[t * DK + a], Ks[t * DK + a], s);
            Inv[t] = s > 0.0f ? 1.0f / s : 0.0f;
        }
        __syncthreads();

        // ---- G = beta_t kappa_t.kappa_j (j < t) and Aq = phi(q_t).kappa_j (j <= t),
        // from raw dot products on the matrix cores: kappa_t.kappa_j =
        // (k_t.k_j)^2 / (|k_t|^2 |k_j|^2); the lifted keys and queries of the chunk
        for (int tile = wave; tile < MT * MT; tile += NWV) {
            const int mt = tile / MT, jt = tile % MT;
            f32x4_t dk = zero4(), dq = zero4();
#pragma unroll
            for (int s4 = 0; s4 < DK / 4; ++s4) {
                const int a = 4 * s4 + g4;
                const float kb = Ks[(16 * jt + c16) * DK + a];
                dk = mfma4(Ks[(16 * mt + c16) * DK + a], kb, dk);
                dq = mfma4(Qs[(16 * mt + c16) * DK + a], kb, dq);
            }
            const int jj = 16 * jt + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * mt + 4 * g4 + r;
                G[t * C + jj] = jj < t ? Bs[t] * (dk[r] * dk[r]) * (Inv[t] * Inv[jj]) : 0.0f;
                Aq[t * C + jj] = jj <= t ? (dq[r] * dq[r]) * Inv[jj] : 0.0f;
            }
        }
        if constexpr (F::PRE) {
            for (int e = tid; e < C * D; e += NT) {
                const int t = e / D, p = e % D;
                const uint32_t pr = pairs[p];
                const int a = pr & 0xff, b = pr >> 8;
                const float sc = a == b ? 1.0f : kSqrt2;
                Kap[e] = Ks[t * DK + a] * Ks[t * DK + b] * (sc * Inv[t]);
                Fq[e] = Qs[t * DK + a] * Qs[t * DK + b] * sc;
            }
        }
        __syncthreads();

        // ---- R = U - K A (tiles of 16 tokens x 16 columns; the second column
        // tile holds only z)
        for (int tile = wave; tile < MT * 2; tile += NWV) {
            const int mt = tile >> 1, col = 16 * (tile & 1) + c16;
            const bool colok = col < kCols;
            f32x4_t acc = zero4();
#pragma unroll 2
            for (int s4 = 0; s4 < D / 4; ++s4) {
                const int p = 4 * s4 + g4;
                acc = mfma4(kappa(16 * mt + c16, p), colok ? St[p * kCols + col] : 0.0f, acc);
            }
            if (colok) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * mt + 4 * g4 + r;
                    R[t * kCols + col] = Us[t * kCols + col] - acc[r];
                }
            }
        }
        // ---- inverses of the diagonal blocks I + N_b (N_b strictly lower, the
        // block's part of G): column j of each inverse by forward substitution
        // (G is complete after the barrier above)
        if (tid >= NT - F::NB * kSub) {
            const int id = tid - (NT - F::NB * kSub);
            const int b = id / kSub, j = id % kSub, r0 = kSub * b;
            float x[kSub];
#pragma unroll
            for (int r = 0; r < kSub; ++r) {
                float s = r == j ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) s = __builtin_fmaf(-G[(r0 + r) * C + r0 + s2], x[s2], s);
                x[r] = s;
            }
#pragma unroll
            for (int r = 0; r < kSub; ++r) TI[(b * kSub + r) * kSub + j] = x[r];
        }
        __syncthreads();

        // ---- P block by block: rhs = beta R - G_{b,<b} P_{<b}, P_b = inv_b rhs
#pragma unroll 1
        for (int b = 0; b < F::NB; ++b) {
            const int r0 = kSub * b;
            for (int e = tid; e < kSub * kCols; e += NT) {
                const int t = r0 + e / kCols, c = e % kCols;
                float s = Bs[t] * R[t * kCols + c];
#pragma unroll 4
                for (int j = 0; j < r0; ++j) s = __builtin_fmaf(-G[t * C + j], P[j * kCols + c], s);
                R[t * kCols + c] = s;
            }
            __syncthreads();
            for (int e = tid; e < kSub * kCols; e += NT) {
                const int r = e / kCols, c = e % kCols;
                float s = 0.0f;
#pragma unroll 4
                for (int j = 0; j < kSub; ++j)
                    s = __builtin_fmaf(TI[(b * kSub + r) * kSub + j], R[(r0 + j) * kCols + c], s);
                P[(r0 + r) * kCols + c] = s;
            }
            __syncthreads();
        }

        // ---- O = phi(Q) A + mask(phi(Q) K^T) P (Aq holds the masked weights)
        for (int tile = wave; tile < MT * 2; tile += NWV) {
            const int mt = tile >> 1, col = 16 * (tile & 1) + c16;
            const bool colok = col < kCols;
            f32x4_t acc = zero4();
#pragma unroll 2
            for (int s4 = 0; s4 < D / 4; ++s4) {
                const int p = 4 * s4 + g4;
                acc = mfma4(phiq(16 * mt + c16, p), colok ? St[p * kCols + col] : 0.0f, acc);
            }
#pragma unroll 2
            for (int s4 = 0; s4 < C / 4; ++s4) {
                const int jj = 4 * s4 + g4;
                acc = mfma4(Aq[(16 * mt + c16) * C + jj], colok ? P[jj * kCols + col] : 0.0f, acc);
            }
            if (colok) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Os[(16 * mt + 4 * g4 + r) * kCols + col] = acc[r];
            }
        }
        __syncthreads();

        // ---- normalise and store; the state gains K^T P (tiles of 16 features
        // x 16 columns; the outputs above were the last reads of the old state)
        for (int e = tid; e < n * kSub; e += NT) {
            const int t = e / kSub, c = e % kSub;
            io<TIn>::st(o, (tok0 + t) * DV + kSub * vt + c, safe_div(Os[t * kCols + c], Os[t * kCols + kSub]));
        }
        for (int tile = wave; tile < FT * 2; tile += NWV) {
            const int ft = tile >> 1, col = 16 * (tile & 1) + c16;
            const bool colok = col < kCols;
            const int pa = 16 * ft + c16;            // this lane's A row (feature)
            f32x4_t acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = 16 * ft + 4 * g4 + r;
                acc[r] = (p < D && colok) ? St[p * kCols + col] : 0.0f;
            }
#pragma unroll 2
            for (int s4 = 0; s4 < C / 4; ++s4) {
                const int t = 4 * s4 + g4;
                acc = mfma4(pa < D ? kappa(t, pa) : 0.0f, colok ? P[t * kCols + col] : 0.0f, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = 16 * ft + 4 * g4 + r;
                if (p < D && colok) St[p * kCols + col] = acc[r];
            }
        }
        __syncthreads();
    }

    if (S_out) {
        for (int e = tid; e < D * kCols; e += NT) {
            const int p = e / kCols, c = e % kCols;
            if (c < kSub) S_out[(bh * D + p) * DV + kSub * vt + c] = St[e];
            else if (vt == 0) z_out[bh * D + p] = St[e];
        }
    }
}

// One decode step per row (block): A += beta kappa (u - kappa^T A), then the
// normalised read. Each thread keeps its rows of the row's state in registers
// between the two reductions (kappa^T A, then phi(q).A).
template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kThreads) void delta_decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ beta, float* __restrict__ S, float* __restrict__ z,
    TIn* __restrict__ o) {
    constexpr int D = DK * (DK + 1) / 2;
    constexpr int C4 = DV / 4;
    constexpr int RG = kThreads / C4;
    constexpr int RPT = (D + RG - 1) / RG;
    __shared__ float fq[D], fk[D], vs[DV], qs[DK], ks[DK];
    __shared__ float4 red[RG][C4];
    __shared__ float zred[kThreads / 64], e4s[DV + 1], ez;

    const size_t row = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < DK) {
        qs[tid] = io<TIn>::ld(q, row * DK + tid);
        ks[tid] = io<TIn>::ld(k, row * DK + tid);
    }
    if (tid < DV) vs[tid] = io<TIn>::ld(v, row * DV + tid);
    __syncthreads();
    float kn2 = 0.0f;
#pragma unroll
    for (int a = 0; a < DK; ++a) kn2 = __builtin_fmaf(ks[a], ks[a], kn2);
    const float inv = kn2 > 0.0f ? 1.0f / kn2 : 0.0f;
    for (int p = tid; p < D; p += kThreads) {
        const uint32_t pr = pack_pair(p, DK);
        const int i = pr & 0xff, j = pr >> 8;
        const float sc = i == j ? 1.0f : kSqrt2;
        fq[p] = sc * (qs[i] * qs[j]);
        fk[p] = sc * (ks[i] * ks[j]) * inv;          // kappa
    }
    __syncthreads();

    const int rg = tid / C4, c4 = tid % C4;
    float4* S4 = reinterpret_cast<float4*>(S + row * (size_t)D * DV);
    float* zr = z + row * (size_t)D;
    float4 cur[RPT];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int p = rg + u * RG;
        if (p < D) {
            cur[u] = S4[p * C4 + c4];
            const float a = fk[p];
            acc.x = __builtin_fmaf(a, cur[u].x, acc.x);
            acc.y = __builtin_fmaf(a, cur[u].y, acc.y);
            acc.z = __builtin_fmaf(a, cur[u].z, acc.z);
            acc.w = __builtin_fmaf(a, cur[u].w, acc.w);
        }
    }
    red[rg][c4] = acc;
    float zpart = 0.0f;
    for (int p = tid; p < D; p += kThreads) zpart = __builtin_fmaf(fk[p], zr[p], zpart);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) zpart += __shfl_xor(zpart, off, 64);
    if ((tid & 63) == 0) zred[tid >> 6] = zpart;
    __syncthreads();
    if (tid < DV) {                               // erase e = kappa^T S
        const int cc = tid / 4, w = tid % 4;
        float s = 0.0f;
        for (int g = 0; g < RG; ++g) {
            const float4 r = red[g][cc];
            s += w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
        }
        e4s[tid] = s;
    }
    if (tid == 0) {
        float s = 0.0f;
#pragma unroll
        for (int u = 0; u < kThreads / 64; ++u) s += zred[u];
        ez = s;
    }
    __syncthreads();

    const float bt = beta[row];
    const float4 d4 = make_float4(bt * (vs[4 * c4] - e4s[4 * c4]), bt * (vs[4 * c4 + 1] - e4s[4 * c4 + 1]),
                                  bt * (vs[4 * c4 + 2] - e4s[4 * c4 + 2]), bt * (vs[4 * c4 + 3] - e4s[4 * c4 + 3]));
    acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int p = rg + u * RG;
        if (p < D) {
            const float a = fk[p], b = fq[p];
            float4 s = cur[u];
            s.x = __builtin_fmaf(a, d4.x, s.x);
            s.y = __builtin_fmaf(a, d4.y, s.y);
            s.z = __builtin_fmaf(a, d4.z, s.z);
            s.w = __builtin_fmaf(a, d4.w, s.w);
            S4[p * C4 + c4] = s;
            acc.x = __builtin_fmaf(b, s.x, acc.x);
            acc.y = __builtin_fmaf(b, s.y, acc.y);
            acc.z = __builtin_fmaf(b, s.z, acc.z);
            acc.w = __builtin_fmaf(b, s.w, acc.w);
        }
    }
    __syncthreads();                              // red is reused
    red[rg][c4] = acc;
    const float dz = bt * (1.0f - ez);
    float dpart = 0.0f;
    for (int p = tid; p < D; p += kThreads) {
        const float zn = __builtin_fmaf(fk[p], dz, zr[p]);
        zr[p] = zn;
        dpart = __builtin_fmaf(fq[p], zn, dpart);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off, 64);
    if ((tid & 63) == 0) zred[tid >> 6] = dpart;
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
        for (int u = 0; u < kThreads / 64; ++u) den += zred[u];
        io<TIn>::st(o, row * DV + tid, safe_div(num, den));
    }
}

template <typename TIn, int DK, int C>
hipError_t launch_fwd_t(const Shape& s, const void* q, const void* k, const void* v,
                        const float* beta, void* o, const float* S0, const float* z0, float* S_out,
                        float* z_out, hipStream_t st) {
    dim3 grid(s.dv / kSub, s.B * s.H);
    delta_fwd_kernel<TIn, DK, C><<<grid, kFwdThreads, 0, st>>>(
        (const TIn*)q, (const TIn*)k, (const TIn*)v, beta, (TIn*)o, S0, z0, S_out, z_out, s.T, s.dv);
    return hipGetLastError();
}

template <typename TIn, int DK>
hipError_t launch_fwd_dk(const Shape& s, const void* q, const void* k, const void* v,
                         const float* beta, void* o, const float* S0, const float* z0,
                         float* S_out, float* z_out, hipStream_t st) {
    switch (s.C) {
        case 16: return launch_fwd_t<TIn, DK, 16>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st);
        case 32: return launch_fwd_t<TIn, DK, 32>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st);
        case 64: return launch_fwd_t<TIn, DK, 64>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st);
    }
    return hipErrorInvalidValue;
}

template <typename TIn, int DK, int DV>
hipError_t launch_dec(const void* q, const void* k, const void* v, const float* beta, float* S,
                      float* z, void* o, int N, hipStream_t st) {
    delta_decode_kernel<TIn, DK, DV><<<N, kThreads, 0, st>>>((const TIn*)q, (const TIn*)k,
                                                             (const TIn*)v, beta, S, z, (TIn*)o);
    return hipGetLastError();
}

template <typename TIn, int DK>
hipError_t launch_dec_dk(const void* q, const void* k, const void* v, const float* beta, float* S,
                         float* z, void* o, int N, int dv, hipStream_t st) {
    switch (dv) {
        case 16: return launch_dec<TIn, DK, 16>(q, k, v, beta, S, z, o, N, st);
        case 32: return launch_dec<TIn, DK, 32>(q, k, v, beta, S, z, o, N, st);
        case 64: return launch_dec<TIn, DK, 64>(q, k, v, beta, S, z, o, N, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool delta_supported(const Shape& s) {
    return (s.dk == 16 || s.dk == 32) && (s.dv == 16 || s.dv == 32 || s.dv == 64) &&
           (s.C == 16 || s.C == 32 || s.C == 64);
}

hipError_t launch_delta_fwd(const Shape& s, const void* q, const void* k, const void* v,
                            const float* beta, void* o, const float* S0, const float* z0,
                            float* S_out, float* z_out, hipStream_t st) {
    if (s.bf16)
        return s.dk == 16 ? launch_fwd_dk<bf16_t, 16>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st)
                          : launch_fwd_dk<bf16_t, 32>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st);
    return s.dk == 16 ? launch_fwd_dk<float, 16>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st)
                      : launch_fwd_dk<float, 32>(s, q, k, v, beta, o, S0, z0, S_out, z_out, st);
}

hipError_t launch_delta_decode(const void* q, const void* k, const void* v, const float* beta,
                               float* S, float* z, void* o, int N, int dk, int dv, bool bf16,
                               hipStream_t st) {
    if (bf16)
        return dk == 16 ? launch_dec_dk<bf16_t, 16>(q, k, v, beta, S, z, o, N, dv, st)
                        : launch_dec_dk<bf16_t, 32>(q, k, v, beta, S, z, o, N, dv, st);
    return dk == 16 ? launch_dec_dk<float, 16>(q, k, v, beta, S, z, o, N, dv, st)
                    : launch_dec_dk<float, 32>(q, k, v, beta, S, z, o, N, dv, st);
}

}  // namespace kata
