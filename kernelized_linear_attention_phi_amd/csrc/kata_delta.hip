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
//     P = T R,   T = (I + diag(beta) L)^-1 diag(beta),   L the strictly lower
//                                      part of K K^T,
//     O = phi(Q) A + mask(phi(Q) K^T) P      (inclusive causal mask),
//     A <- A + K^T P.
// T and the masked weights depend on the chunk's keys, queries and write
// strengths only, so they are formed for every chunk at once by a first kernel
// (delta_prep_kernel, one workgroup per chunk: the inverse of each unit
// lower-triangular 16 x 16 diagonal block by forward substitution, then block
// rows in order). The second kernel (delta_chain_kernel) walks the chunks of one
// (batch, head, value tile) in order and does only the four products above on
// the fp32 matrix cores. A value tile is 15 value columns plus the z column,
// so one 16-column product tile carries both numerator and denominator.
// Scalings: with Inv_t = 1 / |k_t|^2 the first kernel stores diag(Inv) T and
// the mask of (q_t.k_j)^2, so the chain works with the plain lifts phi(k),
// phi(q):  R = U - diag(Inv) phi(K) A,  P' = diag(Inv) T R,
// O = phi(Q) A + mask((Q K^T)^2) P',  A <- A + phi(K)^T P'.
#include "kata_chunk.h"
#include "kata_device.h"
#include "kata_internal.h"
#include "kata_mfma.h"

#include <utility>

namespace kata {

namespace {

constexpr int kThreads = 256;          // decode
constexpr int kPrepThreads = 256;      // per-chunk triangular inverses
constexpr int kChainThreads = 512;     // chunk walk: 8 wavefronts per (head, value tile)
constexpr int kSub = 16;               // rows per block of the triangular solve
constexpr int kTileCols = 16;          // state columns per workgroup: 15 values + z
constexpr int kVals = 15;

// D = A(16x4) * B(4x16) + C in fp32 (v_mfma_f32_16x16x4_f32): fp32 operands,
// fp32 accumulation. Lane (c16, g) supplies A[c16][g] and B[g][c16] and holds
// rows 4g + r of column c16 of the result.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Per-chunk matrices are stored in the layout the chain kernel reads them in as
// matrix-core A operands: element (mt 64 + lane) C/4 + s of a chunk's C x C
// matrix X holds X[16 mt + lane % 16][4 s + lane / 16], so each lane's C/4
// values of one token tile mt are contiguous.

template <int DK, int C>
struct PrepCfg {
    static constexpr int NB = C / kSub;
    static constexpr int MT = C / 16;
    // LDS, in floats
    static constexpr int K_OFF = 0;                     // keys [C][DK]
    static constexpr int Q_OFF = K_OFF + C * DK;        // queries [C][DK]
    static constexpr int INV_OFF = Q_OFF + C * DK;      // 1 / |k_t|^2 [C]
    static constexpr int B_OFF = INV_OFF + C;           // beta [C]
    static constexpr int G_OFF = B_OFF + C;             // beta_t kappa_t.kappa_j, j < t [C][C]
    static constexpr int T_OFF = G_OFF + C * C;         // T [C][C]
    static constexpr int X_OFF = T_OFF + C * C;         // block right-hand sides [16][C]
    static constexpr int TI_OFF = X_OFF + kSub * C;     // diagonal block inverses [NB][16][16]
    static constexpr int FLOATS = TI_OFF + NB * kSub * kSub;
    static_assert(C % kSub == 0 && NB * kSub <= kPrepThreads && MT <= kPrepThreads / 64,
                  "chunk of 16, 32 or 64");
};

// One workgroup of four wavefronts per (chunk, batch*head): writes diag(Inv) T
// and the mask of
// (q_t.k_j)^2 (j <= t) for the chunk, 2 C^2 floats at
// ws + ((bh * NC + chunk) * 2) C^2, in that layout.
template <typename TIn, int DK, int C>
__global__ __launch_bounds__(kPrepThreads) void delta_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ beta,
    float* __restrict__ ws, int T, int NC) {
    using F = PrepCfg<DK, C>;
    constexpr int NT = kPrepThreads;
    __shared__ float sm[F::FLOATS];
    float* Ks = sm + F::K_OFF;
    float* Qs = sm + F::Q_OFF;
    float* Inv = sm + F::INV_OFF;
    float* Bs = sm + F::B_OFF;
    float* G = sm + F::G_OFF;
    float* Tm = sm + F::T_OFF;
    float* X = sm + F::X_OFF;
    float* TI = sm + F::TI_OFF;
    float* Ms = G;                              // the masked weights, once G is done

    const int chunk = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int c0 = chunk * C;
    const int n = min(C, T - c0);
    const size_t tok0 = bh * (size_t)T + c0;
    float* out = ws + (bh * NC + chunk) * (size_t)(2 * C * C);

    // rows past a ragged end are zero: no key, no write, beta 0
    for (int e = tid; e < C * DK; e += NT) {
        const bool ok = e / DK < n;
        Ks[e] = ok ? io<TIn>::ld(k, tok0 * DK + e) : 0.0f;
        Qs[e] = ok ? io<TIn>::ld(q, tok0 * DK + e) : 0.0f;
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

    // G = beta_t kappa_t.kappa_j (j < t), with kappa_t.kappa_j =
    // (k_t.k_j)^2 Inv_t Inv_j; (with X = Q, after the solve) the masked
    // weights (q_t.k_j)^2 (j <= t)
    const int wave = tid >> 6, lane = tid & 63, c16 = lane & 15, g4 = lane >> 4;
    auto gram = [&](const float* X, bool keys) {
        for (int tile = wave; tile < F::MT * F::MT; tile += NT / 64) {
            const int mt = tile / F::MT, jt = tile % F::MT;
            f32x4_t d = zero4();
#pragma unroll
            for (int s4 = 0; s4 < DK / 4; ++s4) {
                const int a = 4 * s4 + g4;
                d = mfma4(X[(16 * mt + c16) * DK + a], Ks[(16 * jt + c16) * DK + a], d);
            }
            const int jj = 16 * jt + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * mt + 4 * g4 + r;
                if (keys) G[t * C + jj] = jj < t ? Bs[t] * (d[r] * d[r]) * (Inv[t] * Inv[jj]) : 0.0f;
                else Ms[t * C + jj] = jj <= t ? d[r] * d[r] : 0.0f;
            }
        }
    };
    gram(Ks, true);
    __syncthreads();

    // inverses of the diagonal blocks I + G_bb: column j of each by forward
    // substitution
    if (tid < F::NB * kSub) {
        const int b = tid / kSub, j = tid % kSub, r0 = kSub * b;
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

    // block rows of (I + G) T = diag(beta) in order,
    // T_b = inv_b (diag(beta)_b - G_{b,<b} T_{<b}), both products on the matrix
    // cores: wavefront w forms column tile w of the block row (T is lower
    // triangular, so tiles right of the diagonal block are zero)
#pragma unroll 1
    for (int b = 0; b < F::NB; ++b) {
        const int r0 = kSub * b;
        const int ct = wave, j = 16 * ct + c16;
        if (ct < F::MT) {
            f32x4_t acc = zero4();
            if (ct < b)
                for (int s4 = 0; s4 < r0 / 4; ++s4)
                    acc = mfma4(G[(r0 + c16) * C + 4 * s4 + g4], Tm[(4 * s4 + g4) * C + j], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = r0 + 4 * g4 + r;
                X[(4 * g4 + r) * C + j] = (t == j ? Bs[t] : 0.0f) - acc[r];
            }
        }
        __syncthreads();
        if (ct < F::MT) {
            f32x4_t acc = zero4();
            if (ct <= b) {
#pragma unroll
                for (int s4 = 0; s4 < kSub / 4; ++s4)
                    acc = mfma4(TI[(b * kSub + c16) * kSub + 4 * s4 + g4], X[(4 * s4 + g4) * C + j], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Tm[(r0 + 4 * g4 + r) * C + j] = acc[r];
        }
        __syncthreads();
    }
    gram(Qs, false);
    __syncthreads();
    // diag(Inv) T and the masked weights, written in the chain kernel's order
    for (int f = tid; f < C * C; f += NT) {
        constexpr int S4 = C / 4;
        const int ln = (f / S4) % 64;
        const int t = 16 * (f / (64 * S4)) + (ln & 15), j = 4 * (f % S4) + (ln >> 4);
        out[f] = Inv[t] * Tm[t * C + j];
        out[C * C + f] = Ms[t * C + j];
    }
}

template <int DK, int C>
struct ChainCfg {
    static constexpr int D = DK * (DK + 1) / 2;
    static constexpr int MT = C / 16;                   // token tiles
    static constexpr int FT = (D + 15) / 16;            // feature tiles
    static constexpr int S4 = C / 4;                    // 4-token steps of a chunk
    // Feature order of the state rows. d_k = 16: circulant, row 16 delta + rho
    // holds the pair (rho, (rho + delta) mod 16) for delta = 0..7 and, for
    // delta = 8, rho = 0..7 (136 rows, every unordered pair once); a lane then
    // lifts its own token's features from one rotated copy of the token in
    // registers with compile-time indices. d_k = 32: the packed row-major
    // order, lifted through a pair table.
    static constexpr bool CIRC = DK == 16;
    // LDS, in floats
    static constexpr int A_OFF = 0;                     // state [D][16] (column 15 = z)
    static constexpr int K_OFF = A_OFF + D * kTileCols; // keys [C][DK]
    static constexpr int Q_OFF = K_OFF + C * DK;        // queries [C][DK]
    static constexpr int U_OFF = Q_OFF + C * DK;        // [v | 1] [C][16]
    static constexpr int R_OFF = U_OFF + C * kTileCols; // R [C][16]
    static constexpr int P_OFF = R_OFF + C * kTileCols; // P' [C][16]
    static constexpr int FLOATS = P_OFF + C * kTileCols;
    static_assert(D % 8 == 0 && MT <= 4, "pairs of 4-feature steps, at most 4 token tiles");
    static_assert(FLOATS * 4 + D * 4 <= 160 * 1024, "fits the LDS of a compute unit");
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }

// Workgroups of one head run on one XCD (so the per-chunk matrices they all
// read stay in that XCD's L2): linear block L -> head 8 (L / (8 NVT)) + L % 8,
// value tile (L / 8) % NVT.
__device__ __forceinline__ void chain_coords(int NVT, int& vt, int& bh) {
    const int L = blockIdx.x;
    bh = 8 * (L / (8 * NVT)) + L % 8;
    vt = (L / 8) % NVT;
}

// Index of the pair (i, j), i <= j, in the packed row-major upper triangle of
// width d.
__device__ __forceinline__ int packed_index(int i, int j, int d) {
    return i * d - i * (i - 1) / 2 + (j - i);
}

// Circulant state row f (d_k = 16) -> its packed feature index.
__device__ __forceinline__ int circ_to_packed(int f) {
    const int delta = f >> 4, rho = f & 15, r2 = (rho + delta) & 15;
    return packed_index(min(rho, r2), max(rho, r2), 16);
}

// Circulant feature 4 S + g of a token whose coordinates a lane of group g holds
// rotated by g (y[m] = x[(m + g) mod 16]): x_rho x_{rho + delta}, scaled by
// sqrt 2 off the diagonal, with delta = S / 4 and rho = 4 (S mod 4) + g.
template <int S>
__device__ __forceinline__ float circ_feature(const float (&y)[16]) {
    constexpr int delta = S / 4, j = S % 4;
    if constexpr (delta == 0) return y[4 * j] * y[4 * j];
    else return y[4 * j] * (kSqrt2 * y[(4 * j + delta) % 16]);
}

// acc (+ acc2 for odd steps) += phi(x) rows of the lane's token against the
// state rows 4 S + g, S = 0 .. D/4 - 1 (d_k = 16).
template <int... S>
__device__ __forceinline__ void circ_products(const float (&y)[16], const float* St, int c16,
                                              int g4, f32x4_t& acc, f32x4_t& acc2,
                                              std::integer_sequence<int, S...>) {
    ((S % 2 == 0 ? (acc = mfma4(circ_feature<S>(y), St[(4 * S + g4) * kTileCols + c16], acc))
                 : (acc2 = mfma4(circ_feature<S>(y), St[(4 * S + g4) * kTileCols + c16], acc2))),
     ...);
}

// One workgroup of 8 wavefronts per (batch*head, value tile of 15 columns + z).
// Wavefronts 0..MT-1 form R and P' of token tile w, wavefronts 4..3+MT the
// outputs of token tile w - 4; feature tiles of the state update are dealt
// round-robin over all eight. The barriers of the chunk loop wait for LDS
// operations only, so the next chunk's loads and this chunk's output stores
// stay in flight across them.
template <typename TIn, int DK, int C>
__global__ __launch_bounds__(kChainThreads) void delta_chain_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ ws, TIn* __restrict__ o, const float* __restrict__ S0,
    const float* __restrict__ z0, float* __restrict__ S_out, float* __restrict__ z_out, int T,
    int DV, int BH, int NVT) {
    using F = ChainCfg<DK, C>;
    constexpr int D = F::D, NT = kChainThreads, S4 = F::S4;
    __shared__ float sm[F::FLOATS];
    __shared__ uint32_t pairs[F::CIRC ? 1 : D];          // packed order: feature -> pair
    float* St = sm + F::A_OFF;
    float* Ks = sm + F::K_OFF;
    float* Qs = sm + F::Q_OFF;
    float* Us = sm + F::U_OFF;
    float* R = sm + F::R_OFF;
    float* P = sm + F::P_OFF;

    int vt, bhi;
    chain_coords(NVT, vt, bhi);
    if (bhi >= BH) return;                     // padding of the head count to 8
    const size_t bh = bhi;
    const int tid = threadIdx.x;
    const int NC = (T + C - 1) / C;
    const int col0 = kVals * vt;
    // state column c of this workgroup: value column col0 + c (c < 15, if it
    // exists) or z (c = 15)
    auto vcol = [&](int c) { return c < kVals && col0 + c < DV; };
    // state row f -> packed feature index
    auto packed = [&](int f) { return F::CIRC ? circ_to_packed(f) : f; };

    if constexpr (!F::CIRC)
        for (int p = tid; p < D; p += NT) pairs[p] = pack_pair(p, DK);
    for (int e = tid; e < D * kTileCols; e += NT) {
        const int f = e / kTileCols, c = e % kTileCols;
        float x = 0.0f;
        if (S0) {
            const int p = packed(f);
            if (c == kVals) x = z0[bh * D + p];
            else if (vcol(c)) x = S0[(bh * D + p) * DV + col0 + c];
        }
        St[e] = x;
    }

    const int wave = tid >> 6, lane = tid & 63, c16 = lane & 15, g4 = lane >> 4;
    const bool rwave = wave < F::MT;                       // forms R, P' of tile wave
    const bool owave = wave >= 4 && wave < 4 + F::MT;      // outputs of tile wave - 4
    const int mt = rwave ? wave : wave - 4;

    // a chunk's inputs are loaded into registers one chunk ahead and staged
    // into LDS once the chunk before is done. The loads are unconditional (their
    // addresses clamped into the chunk's valid rows and the head's columns), so
    // that no branch join makes the wavefront wait for them; rows past a ragged
    // end and columns past d_v are zeroed when staged.
    // The raw input words are kept until then: a conversion right after the
    // load would wait for it.
    constexpr int EK = (C * DK + NT - 1) / NT, EU = (C * kTileCols + NT - 1) / NT;
    TIn nk[EK], nq[EK], nu[EU];
    auto fetch = [&](int c0) {
        const int n = min(C, T - c0);
        const size_t tok0 = bh * (size_t)T + c0;
#pragma unroll
        for (int i = 0; i < EK; ++i) {
            const int e = (tid + i * NT) % (C * DK);
            const int ec = min(e / DK, n - 1) * DK + e % DK;
            nk[i] = k[tok0 * DK + ec];
            nq[i] = q[tok0 * DK + ec];
        }
#pragma unroll
        for (int i = 0; i < EU; ++i) {
            const int e = (tid + i * NT) % (C * kTileCols);
            const int t = min(e / kTileCols, n - 1), col = min(col0 + e % kTileCols, DV - 1);
            nu[i] = v[(tok0 + t) * DV + col];
        }
    };
    // this chunk's T' (R wavefronts) or masked weights (output wavefronts),
    // also loaded one chunk ahead
    float mf[S4], mfn[S4];
    auto fetch_mats = [&](int c, float (&dst)[S4]) {
        if (rwave || owave) {
            const float* src = ws + ((bh * NC + c) * 2 + (owave ? 1 : 0)) * (size_t)(C * C) +
                               (size_t)(mt * 64 + lane) * S4;
#pragma unroll
            for (int s = 0; s < S4; s += 4) {
                const float4 x = *reinterpret_cast<const float4*>(src + s);
                dst[s] = x.x;
                dst[s + 1] = x.y;
                dst[s + 2] = x.z;
                dst[s + 3] = x.w;
            }
        }
    };
    fetch(0);
    fetch_mats(0, mf);
    __syncthreads();

    for (int c = 0; c < NC; ++c) {
        const int c0 = c * C;
        const int n = min(C, T - c0);
        const size_t tok0 = bh * (size_t)T + c0;
        // ---- stage the chunk, start loading the next one (inputs and
        // matrices)
#pragma unroll
        for (int i = 0; i < EK; ++i) {
            const int e = tid + i * NT;
            if (e < C * DK) {
                const bool ok = e / DK < n;
                Ks[e] = ok ? to_f32(nk[i]) : 0.0f;
                Qs[e] = ok ? to_f32(nq[i]) : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < EU; ++i) {
            const int e = tid + i * NT;
            const int t = e / kTileCols, cc = e % kTileCols;
            if (e < C * kTileCols)
                Us[e] = t >= n ? 0.0f : cc == kVals ? 1.0f : vcol(cc) ? to_f32(nu[i]) : 0.0f;
        }
        lds_barrier();
        if (c + 1 < NC) {
            fetch(c0 + C);
            fetch_mats(c + 1, mfn);
        }

        // ---- phase 1: R = U - diag(Inv) phi(K) A (R wavefronts) and the
        // inter-chunk part phi(Q) A of the outputs (output wavefronts); both
        // read the state before the chunk. Lane (c16, g) lifts token
        // 16 mt + c16 itself.
        f32x4_t oacc = zero4();
        if (rwave || owave) {
            const float* xr = (rwave ? Ks : Qs) + (16 * mt + c16) * DK;
            // two accumulators so that consecutive products do not wait on
            // each other
            f32x4_t acc = zero4(), acc2 = zero4();
            float nrm = 0.0f;
            if constexpr (F::CIRC) {
                float y[16];
#pragma unroll
                for (int m = 0; m < 16; ++m) y[m] = xr[(m + g4) & 15];
#pragma unroll
                for (int m = 0; m < 16; ++m) nrm = __builtin_fmaf(y[m], y[m], nrm);
                circ_products(y, St, c16, g4, acc, acc2, std::make_integer_sequence<int, D / 4>{});
            } else {
#pragma unroll
                for (int a = 0; a < DK; ++a) nrm = __builtin_fmaf(xr[a], xr[a], nrm);
#pragma unroll 2
                for (int s4 = 0; s4 < D / 4; s4 += 2) {
                    const int p = 4 * s4 + g4;
                    const uint32_t pr = pairs[p], pr2 = pairs[p + 4];
                    const float a = xr[pr & 0xff] * xr[pr >> 8] * ((pr & 0xff) == (pr >> 8) ? 1.0f : kSqrt2);
                    const float a2 = xr[pr2 & 0xff] * xr[pr2 >> 8] * ((pr2 & 0xff) == (pr2 >> 8) ? 1.0f : kSqrt2);
                    acc = mfma4(a, St[p * kTileCols + c16], acc);
                    acc2 = mfma4(a2, St[(p + 4) * kTileCols + c16], acc2);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += acc2[r];
            if (rwave) {
                const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;      // of token 16 mt + c16
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 16 * mt + 4 * g4 + r;
                    const float inv_r = __shfl(inv, 4 * g4 + r, 64);
                    R[tr * kTileCols + c16] = Us[tr * kTileCols + c16] - inv_r * acc[r];
                }
            } else {
                oacc = acc;
            }
        }
        lds_barrier();

        // ---- phase 2: P' = diag(Inv) T R (T lower triangular: token tile mt
        // needs the first 16 (mt + 1) tokens)
        if (rwave) {
            f32x4_t acc = zero4();
#pragma unroll
            for (int s = 0; s < S4; ++s)
                if (s < 4 * (mt + 1)) acc = mfma4(mf[s], R[(4 * s + g4) * kTileCols + c16], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) P[(16 * mt + 4 * g4 + r) * kTileCols + c16] = acc[r];
        }
        lds_barrier();

        // ---- phase 3: the intra-chunk part mask((Q K^T)^2) P' of the outputs,
        // normalise and store (output wavefronts); the state gains phi(K)^T P'
        // (feature tiles round-robin; the last reads of the old state were in
        // phase 1)
        if (owave) {
#pragma unroll
            for (int s = 0; s < S4; ++s)
                if (s < 4 * (mt + 1)) oacc = mfma4(mf[s], P[(4 * s + g4) * kTileCols + c16], oacc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float den = __shfl(oacc[r], 16 * g4 + kVals, 64);
                const int t = 16 * mt + 4 * g4 + r;
                if (t < n && vcol(c16))
                    io<TIn>::st(o, (tok0 + t) * DV + col0 + c16, safe_div(oacc[r], den));
            }
        }
        for (int ft = wave; ft < F::FT; ft += NT / 64) {
            // this lane's A row: state row (feature) 16 ft + c16 = pair (a, b)
            const int f = 16 * ft + c16;
            int a = 0, b = 0;
            float sc = 0.0f;
            if (f < D) {
                if constexpr (F::CIRC) {
                    a = c16;
                    b = (c16 + ft) & 15;
                    sc = ft == 0 ? 1.0f : kSqrt2;
                } else {
                    const uint32_t pr = pairs[f];
                    a = pr & 0xff;
                    b = pr >> 8;
                    sc = a == b ? 1.0f : kSqrt2;
                }
            }
            f32x4_t acc, acc2 = zero4();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = 16 * ft + 4 * g4 + r;
                acc[r] = p < D ? St[p * kTileCols + c16] : 0.0f;
            }
#pragma unroll 4
            for (int s4 = 0; s4 < S4; s4 += 2) {
                const int t = 4 * s4 + g4;
                acc = mfma4(Ks[t * DK + a] * Ks[t * DK + b] * sc, P[t * kTileCols + c16], acc);
                acc2 = mfma4(Ks[(t + 4) * DK + a] * Ks[(t + 4) * DK + b] * sc,
                             P[(t + 4) * kTileCols + c16], acc2);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = 16 * ft + 4 * g4 + r;
                if (p < D) St[p * kTileCols + c16] = acc[r] + acc2[r];
            }
        }
#pragma unroll
        for (int s = 0; s < S4; ++s) mf[s] = mfn[s];
        lds_barrier();
    }

    if (S_out) {
        for (int e = tid; e < D * kTileCols; e += NT) {
            const int f = e / kTileCols, c = e % kTileCols;
            const int p = packed(f);
            if (c == kVals) {
                if (vt == 0) z_out[bh * D + p] = St[e];
            } else if (vcol(c)) {
                S_out[(bh * D + p) * DV + col0 + c] = St[e];
            }
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
                        float* z_out, float* ws, hipStream_t st) {
    const int BH = s.B * s.H;
    const int NC = (s.T + C - 1) / C;
    delta_prep_kernel<TIn, DK, C><<<dim3(NC, BH), kPrepThreads, 0, st>>>(
        (const TIn*)q, (const TIn*)k, beta, ws, s.T, NC);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int NVT = (s.dv + kVals - 1) / kVals;
    const int blocks = NVT * 8 * ((BH + 7) / 8);
    delta_chain_kernel<TIn, DK, C><<<blocks, kChainThreads, 0, st>>>(
        (const TIn*)q, (const TIn*)k, (const TIn*)v, ws, (TIn*)o, S0, z0, S_out, z_out, s.T, s.dv,
        BH, NVT);
    return hipGetLastError();
}

template <typename TIn, int DK>
hipError_t launch_fwd_dk(const Shape& s, const void* q, const void* k, const void* v,
                         const float* beta, void* o, const float* S0, const float* z0,
                         float* S_out, float* z_out, float* ws, hipStream_t st) {
    switch (s.C) {
        case 16: return launch_fwd_t<TIn, DK, 16>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st);
        case 32: return launch_fwd_t<TIn, DK, 32>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st);
        case 64: return launch_fwd_t<TIn, DK, 64>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st);
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

size_t delta_workspace_bytes(const Shape& s) {
    const size_t NC = (size_t)(s.T + s.C - 1) / s.C;
    return (size_t)s.B * s.H * NC * 2 * s.C * s.C * sizeof(float);
}

hipError_t launch_delta_fwd(const Shape& s, const void* q, const void* k, const void* v,
                            const float* beta, void* o, const float* S0, const float* z0,
                            float* S_out, float* z_out, float* ws, hipStream_t st) {
    if (s.bf16)
        return s.dk == 16 ? launch_fwd_dk<bf16_t, 16>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st)
                          : launch_fwd_dk<bf16_t, 32>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st);
    return s.dk == 16 ? launch_fwd_dk<float, 16>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st)
                      : launch_fwd_dk<float, 32>(s, q, k, v, beta, o, S0, z0, S_out, z_out, ws, st);
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
