// Fused bf16 chunked-state forward for d_k = 16 on gfx950 matrix cores.
//
// Method (KATA explainers, gist.science, technical summary 2.3; the paper's
// abstract): the sequence is cut into chunks of C positions; each output is the
// masked intra-chunk term plus phi(Q_c) times the prefix of chunk states; the
// prefix is propagated by an associative scan. Here one wavefront owns a
// segment of G consecutive chunks of one (batch, head) and carries the running
// state S = sum phi(k) v^T (and z = sum phi(k)) in its matrix-core accumulators
// across the segment, so only one state per segment touches HBM:
//   kata_seg_state16 : segment totals         (phi(K)^T [V | 1] on MFMA)
//   (scan kernel)    : exclusive prefix over segments of each head
//   kata_fwd16       : per chunk, intra (QK^T -> square -> mask -> A.V) and inter
//                      (phi(Q).S) on MFMA into one accumulator, normalise,
//                      store, then S += phi(K)^T [V | 1].
//
// Internal feature order ("circulant"). The D = 136 unique products x_a x_b are
// arranged as 9 tiles of 16 rows: tile delta (0..8), row rho (0..15) holds
// x_rho * x_{(rho+delta) mod 16}. Every unordered pair appears once, except
// tile 8 rows 8..15, which repeat rows 0..7 and are kept at zero. The factor 2
// of an off-diagonal pair (sqrt 2 on each side in the packed layout) sits on
// the query side, so the internal state holds plain sums of k_a k_b v. With
// this order a lane's row is fixed, so phi(K) needs one DPP row rotation per
// tile and phi(Q) is built from a per-lane rotated copy of q: no LDS traffic
// for either lift.
//
// Denominators ride along as a fifth value tile whose first column is 1 (the
// "ones" tile): z = phi(K)^T 1, phi(Q).z and sum_j A_tj come out of the same
// MFMAs as the numerators.
#include "kata_device.h"
#include "kata_internal.h"
#include "kata_mfma.h"

#include <algorithm>

namespace kata {

namespace {

constexpr int DK = 16;
constexpr int NMT = 9;                  // feature tiles (delta = 0..8)

template <int DV, int C>
struct Cfg {
    static constexpr int NTV = DV / 16;           // value tiles
    static constexpr int NT = NTV + 1;            // + ones tile
    static constexpr int TT = C / 16;             // query tiles per chunk
    static constexpr int KS = C / 32;             // 32-token K-steps per chunk
    static constexpr int QB = C * DK * 2;         // bytes of a q or k chunk
    static constexpr int VB = C * DV * 2;         // bytes of a v chunk
    static constexpr int BUF = 2 * QB + VB;       // one chunk buffer
    static constexpr int NLQKV = BUF / 1024;      // 1 KB async loads: q, k, v
    static constexpr int NLKV = (QB + VB) / 1024; // k, v only
    static constexpr int NSTORE = TT * NTV;       // 8-byte output stores per chunk
};

// Register arrays passed by reference (alias templates keep the declarations
// unambiguous).
template <int DV, int C> using StateRegs = f32x4_t[NMT][Cfg<DV, C>::NT];
template <int DV, int C> using KTRegs = f32x4_t[Cfg<DV, C>::TT];
template <int DV, int C> using KRegs = u32x2_t[Cfg<DV, C>::TT];
template <int DV, int C> using VRegs = u32x4_t[Cfg<DV, C>::KS][Cfg<DV, C>::NTV];

struct Lane {
    int lane, c16, g;
    __device__ Lane() : lane(threadIdx.x & 63), c16(threadIdx.x & 15), g((threadIdx.x >> 4) & 3) {}
};

// Constant operands. ones: column (or row) 0 of the ones tile = 1 on every slot.
__device__ __forceinline__ u32x4_t ones_op(const Lane& L) {
    const uint32_t w = L.c16 == 0 ? 0x3f803f80u : 0u;   // bf16 1.0 twice
    return u32x4_t{w, w, w, w};
}
// B operand of 16x16x32 selecting value column c16 + 16h of a 32-column block:
// slot (g, s) stands for column 8g + s.
__device__ __forceinline__ u32x4_t select32(const Lane& L, int h) {
    u32x4_t r;
    const int want = L.c16 + 16 * h;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int s0 = 8 * L.g + 2 * p;
        r[p] = (s0 == want ? 0x3f80u : 0u) | (s0 + 1 == want ? 0x3f800000u : 0u);
    }
    return r;
}
// B operand of 16x16x16 = identity: slot (g, s) stands for row 4g + s.
__device__ __forceinline__ u32x2_t ident16(const Lane& L) {
    u32x2_t r;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int s0 = 4 * L.g + 2 * p;
        r[p] = (s0 == L.c16 ? 0x3f80u : 0u) | (s0 + 1 == L.c16 ? 0x3f800000u : 0u);
    }
    return r;
}

// ---- chunk staging: q | k | v of one chunk, row-major as in HBM -------------

// Full chunk: 1 KB direct-to-LDS loads (lane l moves bytes [16l, 16l+16)).
template <int DV, int C>
__device__ __forceinline__ void stage_async(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                            size_t tok0, char* buf, bool with_q, const Lane& L) {
    using F = Cfg<DV, C>;
    const char* gq = reinterpret_cast<const char*>(q + tok0 * DK);
    const char* gk = reinterpret_cast<const char*>(k + tok0 * DK);
    const char* gv = reinterpret_cast<const char*>(v + tok0 * DV);
    if (with_q) {
#pragma unroll
        for (int i = 0; i < F::QB / 1024; ++i)
            __builtin_amdgcn_global_load_lds(gq + i * 1024 + L.lane * 16,
                                             (lds_void_t*)(buf + i * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < F::QB / 1024; ++i)
        __builtin_amdgcn_global_load_lds(gk + i * 1024 + L.lane * 16,
                                         (lds_void_t*)(buf + F::QB + i * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < F::VB / 1024; ++i)
        __builtin_amdgcn_global_load_lds(gv + i * 1024 + L.lane * 16,
                                         (lds_void_t*)(buf + 2 * F::QB + i * 1024), 16, 0, 0);
}

// Ragged chunk (n < C valid positions): bounded loads, zero fill, then LDS.
template <int DV, int C>
__device__ __forceinline__ void stage_ragged(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                             size_t tok0, int n, char* buf, bool with_q,
                                             const Lane& L) {
    using F = Cfg<DV, C>;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t* gq = reinterpret_cast<const u32x4_t*>(q + tok0 * DK);
    const u32x4_t* gk = reinterpret_cast<const u32x4_t*>(k + tok0 * DK);
    const u32x4_t* gv = reinterpret_cast<const u32x4_t*>(v + tok0 * DV);
    u32x4_t* lq = reinterpret_cast<u32x4_t*>(buf);
    u32x4_t* lk = reinterpret_cast<u32x4_t*>(buf + F::QB);
    u32x4_t* lv = reinterpret_cast<u32x4_t*>(buf + 2 * F::QB);
    constexpr int QU = F::QB / 16, VU = F::VB / 16;       // 16-byte units
    constexpr int QPR = DK * 2 / 16, VPR = DV * 2 / 16;   // units per row
    for (int u = L.lane; u < QU; u += 64) {
        const bool ok = u / QPR < n;
        if (with_q) lq[u] = ok ? gq[u] : zero;
        lk[u] = ok ? gk[u] : zero;
    }
    for (int u = L.lane; u < VU; u += 64) lv[u] = (u / VPR < n) ? gv[u] : zero;
    compiler_fence();
}

// ---- per-chunk fragments ----------------------------------------------------

// V^T fragments: vop[m][nt] = 8 values v[token][16nt + c16] for the tokens of
// K-step m in slot order s -> 32m + 16(s/4) + 4g + s%4. Built by multiplying
// row-major V blocks with selection matrices (the accumulator layout performs
// the transpose), so V never needs a transposed copy.
template <int DV, int C>
__device__ __forceinline__ void v_fragments(const bf16_t* bv, VRegs<DV, C>& vop, const Lane& L) {
    using F = Cfg<DV, C>;
#pragma unroll
    for (int m = 0; m < F::KS; ++m) {
        if constexpr (F::NTV % 2 == 0) {
            const u32x4_t sel0 = select32(L, 0), sel1 = select32(L, 1);
#pragma unroll
            for (int ntp = 0; ntp < F::NTV / 2; ++ntp) {
                f32x4_t t[2][2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(
                        bv + (32 * m + 16 * h + L.c16) * DV + 32 * ntp + 8 * L.g);
                    t[h][0] = mma32(vf, sel0, zero4());
                    t[h][1] = mma32(vf, sel1, zero4());
                }
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    vop[m][2 * ntp + e] = u32x4_t{pk2(t[0][e][0], t[0][e][1]), pk2(t[0][e][2], t[0][e][3]),
                                                  pk2(t[1][e][0], t[1][e][1]), pk2(t[1][e][2], t[1][e][3])};
            }
        } else {
            static_assert(F::NTV == 1, "odd value-tile count is only 1");
            const u32x2_t id = ident16(L);
            f32x4_t t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x2_t vf = *reinterpret_cast<const u32x2_t*>(
                    bv + (32 * m + 16 * h + L.c16) * DV + 4 * L.g);
                t[h] = mma16(vf, id, zero4());
            }
            vop[m][0] = u32x4_t{pk2(t[0][0], t[0][1]), pk2(t[0][2], t[0][3]),
                                pk2(t[1][0], t[1][1]), pk2(t[1][2], t[1][3])};
        }
    }
}

// S += phi(K_c)^T [V_c | 1]. KT[jb][r] = k[16jb + 4g + r][c16] (fp32).
template <int DV, int C>
__device__ __forceinline__ void state_update(StateRegs<DV, C>& S, const KTRegs<DV, C>& KT,
                                             const VRegs<DV, C>& vop, const Lane& L) {
    using F = Cfg<DV, C>;
    const u32x4_t ones = ones_op(L);
    const bool upper = L.c16 >= 8;
#pragma unroll
    for (int m = 0; m < F::KS; ++m) {
        float ka[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) ka[s] = KT[2 * m + s / 4][s % 4];
#pragma unroll
        for (int d = 0; d < NMT; ++d) {
            float f[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                float b;
                if (d == 0) b = ka[s];
                else if (d == 1) b = row_fetch<1>(ka[s]);
                else if (d == 2) b = row_fetch<2>(ka[s]);
                else if (d == 3) b = row_fetch<3>(ka[s]);
                else if (d == 4) b = row_fetch<4>(ka[s]);
                else if (d == 5) b = row_fetch<5>(ka[s]);
                else if (d == 6) b = row_fetch<6>(ka[s]);
                else if (d == 7) b = row_fetch<7>(ka[s]);
                else b = row_fetch<8>(ka[s]);
                f[s] = ka[s] * b;
                if (d == 8 && upper) f[s] = 0.0f;          // repeated pairs stay zero
            }
            const u32x4_t fk = {pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7])};
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt) S[d][nt] = mma32(fk, vop[m][nt], S[d][nt]);
            S[d][F::NTV] = mma32(fk, ones, S[d][F::NTV]);
            // keep one tile's lift in flight at a time (bounds register pressure;
            // the matrix core still overlaps the next tile's VALU work)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int DV, int C>
__device__ __forceinline__ void k_fragments(const bf16_t* bk, KRegs<DV, C>& kf, KTRegs<DV, C>& KT,
                                            const Lane& L) {
    using F = Cfg<DV, C>;
    const u32x2_t id = ident16(L);
#pragma unroll
    for (int jb = 0; jb < F::TT; ++jb) {
        kf[jb] = *reinterpret_cast<const u32x2_t*>(bk + (16 * jb + L.c16) * DK + 4 * L.g);
        KT[jb] = mma16(kf[jb], id, zero4());
    }
}

// ---- state records -----------------------------------------------------------
// A record holds one state in accumulator order: S part at
// ((tile * NTV + nt) * 64 + lane) * 4 + r, then the z column (ones tile, column
// 0) at NMT*NTV*256 + tile*16 + 4g + r.

template <int DV, int C>
__device__ __forceinline__ void record_store(float* rec, const StateRegs<DV, C>& S, const Lane& L) {
    using F = Cfg<DV, C>;
    f32x4_t* r4 = reinterpret_cast<f32x4_t*>(rec);
#pragma unroll
    for (int d = 0; d < NMT; ++d)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) r4[(d * F::NTV + nt) * 64 + L.lane] = S[d][nt];
    if (L.c16 == 0) {
#pragma unroll
        for (int d = 0; d < NMT; ++d) r4[NMT * F::NTV * 64 + d * 4 + L.g] = S[d][F::NTV];
    }
}

template <int DV, int C>
__device__ __forceinline__ void record_load(const float* rec, StateRegs<DV, C>& S, const Lane& L) {
    using F = Cfg<DV, C>;
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(rec);
#pragma unroll
    for (int d = 0; d < NMT; ++d)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) S[d][nt] = r4[(d * F::NTV + nt) * 64 + L.lane];
#pragma unroll
    for (int d = 0; d < NMT; ++d)
        S[d][F::NTV] = L.c16 == 0 ? r4[NMT * F::NTV * 64 + d * 4 + L.g] : zero4();
}

// ---- kernels -------------------------------------------------------------------

template <int DV, int C>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void kata_seg_state16(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                      float* __restrict__ rec, int T, int NC, int G, int NSEG) {
    using F = Cfg<DV, C>;
    __shared__ __attribute__((aligned(16))) char lds[2 * F::BUF];
    const Lane L;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int c0 = seg * G, c1 = min(NC, c0 + G);
    f32x4_t S[NMT][F::NT];
#pragma unroll
    for (int d = 0; d < NMT; ++d)
#pragma unroll
        for (int nt = 0; nt < F::NT; ++nt) S[d][nt] = zero4();

    auto stage = [&](int c, char* buf) -> bool {
        const int n = min(C, T - c * C);
        const size_t tok0 = bh * T + (size_t)c * C;
        if (n == C) { stage_async<DV, C>(nullptr, k, v, tok0, buf, false, L); return true; }
        stage_ragged<DV, C>(nullptr, k, v, tok0, n, buf, false, L);
        return false;
    };
    stage(c0, lds);
    for (int c = c0; c < c1; ++c) {
        char* buf = lds + ((c - c0) & 1) * F::BUF;
        const bool more = c + 1 < c1;
        const bool async_next = more && stage(c + 1, lds + ((c + 1 - c0) & 1) * F::BUF);
        if (async_next) wait_vmcnt<F::NLKV>(); else wait_vmcnt<0>();
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::QB);
        u32x2_t kf[F::TT];
        f32x4_t KT[F::TT];
        u32x4_t vop[F::KS][F::NTV];
        k_fragments<DV, C>(bk, kf, KT, L);
        v_fragments<DV, C>(bv, vop, L);
        state_update<DV, C>(S, KT, vop, L);
        compiler_fence();
    }
    record_store<DV, C>(rec + (bh * NSEG + seg) * (size_t)(NMT * F::NTV * 256 + NMT * 16), S, L);
}

template <int DV, int C, bool CAUSAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void kata_fwd16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, const float* __restrict__ prefix,
                bf16_t* __restrict__ o, int T, int NC, int G, int NSEG) {
    using F = Cfg<DV, C>;
    constexpr int REC = NMT * F::NTV * 256 + NMT * 16;
    __shared__ __attribute__((aligned(16))) char lds[2 * F::BUF];
    const Lane L;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int c0 = seg * G, c1 = min(NC, c0 + G);

    f32x4_t S[NMT][F::NT];
    record_load<DV, C>(prefix + (CAUSAL ? bh * NSEG + seg : bh) * (size_t)REC, S, L);

    auto stage = [&](int c, char* buf) -> bool {
        const int n = min(C, T - c * C);
        const size_t tok0 = bh * T + (size_t)c * C;
        if (n == C) { stage_async<DV, C>(q, k, v, tok0, buf, true, L); return true; }
        stage_ragged<DV, C>(q, k, v, tok0, n, buf, true, L);
        return false;
    };
    stage(c0, lds);
    bool stores_pending = false;
    for (int c = c0; c < c1; ++c) {
        char* buf = lds + ((c - c0) & 1) * F::BUF;
        const int n = min(C, T - c * C);
        const bool more = c + 1 < c1;
        const bool async_next = more && stage(c + 1, lds + ((c + 1 - c0) & 1) * F::BUF);
        // wait for this chunk's staging; the newer loads (next chunk) and the
        // previous chunk's output stores (issued after this chunk's loads) may
        // stay in flight
        if (async_next) {
            if (stores_pending) wait_vmcnt<F::NLQKV + F::NSTORE>(); else wait_vmcnt<F::NLQKV>();
        } else {
            if (stores_pending) wait_vmcnt<F::NSTORE>(); else wait_vmcnt<0>();
        }
        const bf16_t* bq = reinterpret_cast<const bf16_t*>(buf);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::QB);

        // K rows and V^T fragments for the intra term; the state update below
        // rebuilds its own copies from the (still resident) LDS buffer so that
        // none of them stays live across the output phase.
        u32x2_t kf[F::TT];
        u32x4_t vop[F::KS][F::NTV];
        if (CAUSAL) {
#pragma unroll
            for (int jb = 0; jb < F::TT; ++jb)
                kf[jb] = *reinterpret_cast<const u32x2_t*>(bk + (16 * jb + L.c16) * DK + 4 * L.g);
            v_fragments<DV, C>(bv, vop, L);
        }
        __builtin_amdgcn_sched_barrier(0);

        // Query tiles are processed in groups of TH (two tiles = 32 rows) to
        // bound the accumulator and rotated-query registers.
        constexpr int TH = F::TT < 2 ? F::TT : 2;
        bf16_t* oc = o + (bh * T + (size_t)c * C) * DV;
#pragma unroll
        for (int t0 = 0; t0 < F::TT; t0 += TH) {
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t num[F::NT][TH];
#pragma unroll
            for (int nt = 0; nt < F::NT; ++nt)
#pragma unroll
                for (int u = 0; u < TH; ++u) num[nt][u] = zero4();

            // query rows of this lane: t = 16tt + c16; q rotated by 4g lanes
            float qr[TH][16];
#pragma unroll
            for (int u = 0; u < TH; ++u) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const u32x2_t piece = *reinterpret_cast<const u32x2_t*>(
                        bq + (16 * (t0 + u) + L.c16) * DK + 4 * ((L.g + a) & 3));
                    qr[u][4 * a + 0] = lo_bf16(piece[0]);
                    qr[u][4 * a + 1] = hi_bf16(piece[0]);
                    qr[u][4 * a + 2] = lo_bf16(piece[1]);
                    qr[u][4 * a + 3] = hi_bf16(piece[1]);
                }
            }

            // ---- intra-chunk term: A = (Q K^T)^2 masked to j <= t, num += A [V | 1]
            if (CAUSAL) {
                const u32x4_t ones = ones_op(L);
#pragma unroll
                for (int u = 0; u < TH; ++u) {
                    const int tt = t0 + u;
                    const u32x2_t qf = *reinterpret_cast<const u32x2_t*>(
                        bq + (16 * tt + L.c16) * DK + 4 * L.g);
                    const int t = 16 * tt + L.c16;
#pragma unroll
                    for (int m = 0; m <= tt / 2; ++m) {
                        const bool diag = 32 * m + 31 > 16 * tt;
                        float w[8];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            // rows j = 16(2m+h) + 4g + r, column t
                            const f32x4_t st = mma16(kf[2 * m + h], qf, zero4());
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int j = 32 * m + 16 * h + 4 * L.g + r;
                                const float x = st[r] * st[r];
                                w[4 * h + r] = (!diag || j <= t) ? x : 0.0f;
                            }
                        }
                        const u32x4_t at = {pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]),
                                            pk2(w[6], w[7])};
#pragma unroll
                        for (int nt = 0; nt < F::NTV; ++nt) num[nt][u] = mma32(vop[m][nt], at, num[nt][u]);
                        num[F::NTV][u] = mma32(ones, at, num[F::NTV][u]);
                    }
                }
            }

            __builtin_amdgcn_sched_barrier(0);
            // ---- inter-chunk term: num += S^T phi(Q)^T over the 9 feature tiles
#pragma unroll
            for (int m = 0; m < 4; ++m) {             // tiles (2m, 2m+1)
                u32x4_t sop[F::NT];
#pragma unroll
                for (int nt = 0; nt < F::NT; ++nt)
                    sop[nt] = u32x4_t{pk2(S[2 * m][nt][0], S[2 * m][nt][1]),
                                      pk2(S[2 * m][nt][2], S[2 * m][nt][3]),
                                      pk2(S[2 * m + 1][nt][0], S[2 * m + 1][nt][1]),
                                      pk2(S[2 * m + 1][nt][2], S[2 * m + 1][nt][3])};
#pragma unroll
                for (int u = 0; u < TH; ++u) {
                    float f[8];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int d = 2 * m + h;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            f[4 * h + r] = d == 0 ? qr[u][r] * qr[u][r]
                                                  : (2.0f * qr[u][r]) * qr[u][(r + d) & 15];
                    }
                    const u32x4_t fq = {pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7])};
#pragma unroll
                    for (int nt = 0; nt < F::NT; ++nt) num[nt][u] = mma32(sop[nt], fq, num[nt][u]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            {                                         // tile 8 (half K-step)
                u32x2_t sop[F::NT];
#pragma unroll
                for (int nt = 0; nt < F::NT; ++nt)
                    sop[nt] = u32x2_t{pk2(S[8][nt][0], S[8][nt][1]), pk2(S[8][nt][2], S[8][nt][3])};
#pragma unroll
                for (int u = 0; u < TH; ++u) {
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) f[r] = (2.0f * qr[u][r]) * qr[u][(r + 8) & 15];
                    const u32x2_t fq = {pk2(f[0], f[1]), pk2(f[2], f[3])};
#pragma unroll
                    for (int nt = 0; nt < F::NT; ++nt) num[nt][u] = mma16(sop[nt], fq, num[nt][u]);
                }
            }

            __builtin_amdgcn_sched_barrier(0);
            // ---- normalise and store: o = num / den (den = row 0 of the ones tile)
#pragma unroll
            for (int u = 0; u < TH; ++u) {
                const int t = 16 * (t0 + u) + L.c16;
                const float den = __shfl(num[F::NTV][u][0], L.c16, 64);
                const float y = 1.0f / den;           // correctly rounded reciprocal
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) {
                    float ov[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // Markstein: with y = RN(1/den), q0 + RN(num - q0 den) y = RN(num/den)
                        const float x = num[nt][u][r];
                        const float q0 = x * y;
                        const float e = __builtin_fmaf(-q0, den, x);
                        const float qq = __builtin_fmaf(e, y, q0);
                        ov[r] = den != 0.0f ? qq : 0.0f;
                    }
                    if (t < n)
                        *reinterpret_cast<u32x2_t*>(oc + (size_t)t * DV + 16 * nt + 4 * L.g) =
                            u32x2_t{pk2(ov[0], ov[1]), pk2(ov[2], ov[3])};
                }
            }
        }
        stores_pending = true;

        // ---- running state: S += phi(K_c)^T [V_c | 1]
        __builtin_amdgcn_sched_barrier(0);
        if (CAUSAL) {
            u32x2_t kf2[F::TT];
            f32x4_t KT[F::TT];
            u32x4_t vop2[F::KS][F::NTV];
            k_fragments<DV, C>(bk, kf2, KT, L);
            v_fragments<DV, C>(bv, vop2, L);
            state_update<DV, C>(S, KT, vop2, L);
        }
        compiler_fence();
    }
}

template <int DV, int C>
hipError_t launch_dv_c(const Shape& s, const void* q, const void* k, const void* v,
                       float* rec, const float* prefix, void* o, int causal, int G, int NSEG,
                       bool state_only, hipStream_t st) {
    dim3 grid(NSEG, s.B * s.H);
    if (state_only) {
        kata_seg_state16<DV, C><<<grid, 64, 0, st>>>((const bf16_t*)k, (const bf16_t*)v, rec,
                                                      s.T, s.NC, G, NSEG);
    } else if (causal) {
        kata_fwd16<DV, C, true><<<grid, 64, 0, st>>>((const bf16_t*)q, (const bf16_t*)k,
                                                      (const bf16_t*)v, prefix, (bf16_t*)o, s.T,
                                                      s.NC, G, NSEG);
    } else {
        kata_fwd16<DV, C, false><<<grid, 64, 0, st>>>((const bf16_t*)q, (const bf16_t*)k,
                                                       (const bf16_t*)v, prefix, (bf16_t*)o, s.T,
                                                       s.NC, G, NSEG);
    }
    return hipGetLastError();
}

template <int C>
hipError_t launch_c(const Shape& s, const void* q, const void* k, const void* v, float* rec,
                    const float* prefix, void* o, int causal, int G, int NSEG, bool state_only,
                    hipStream_t st) {
    switch (s.dv) {
        case 16: return launch_dv_c<16, C>(s, q, k, v, rec, prefix, o, causal, G, NSEG, state_only, st);
        case 32: return launch_dv_c<32, C>(s, q, k, v, rec, prefix, o, causal, G, NSEG, state_only, st);
        case 64: return launch_dv_c<64, C>(s, q, k, v, rec, prefix, o, causal, G, NSEG, state_only, st);
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch(const Shape& s, const void* q, const void* k, const void* v, float* rec,
                    const float* prefix, void* o, int causal, int G, int NSEG, bool state_only,
                    hipStream_t st) {
    switch (s.C) {
        case 32: return launch_c<32>(s, q, k, v, rec, prefix, o, causal, G, NSEG, state_only, st);
        case 64: return launch_c<64>(s, q, k, v, rec, prefix, o, causal, G, NSEG, state_only, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma16_supported(const Shape& s) {
    return s.bf16 && s.dk == 16 && (s.C == 32 || s.C == 64) &&
           (s.dv == 16 || s.dv == 32 || s.dv == 64);
}

int mfma16_record_floats(int dv) { return NMT * (dv / 16) * 256 + NMT * 16; }

hipError_t launch_seg_state16(const Shape& s, const void* k, const void* v, float* rec, int G,
                              int NSEG, hipStream_t st) {
    return dispatch(s, nullptr, k, v, rec, nullptr, nullptr, 1, G, NSEG, true, st);
}

hipError_t launch_fwd16(const Shape& s, const void* q, const void* k, const void* v,
                        const float* prefix, void* o, int causal, int G, int NSEG,
                        hipStream_t st) {
    return dispatch(s, q, k, v, nullptr, prefix, o, causal, G, NSEG, false, st);
}

// ---- record <-> packed state conversion ------------------------------------

namespace {

// Internal record element -> (packed feature index, value column, scale), or -1
// for the repeated (always zero) rows.
__device__ __forceinline__ int record_to_packed(int idx, int NTV, int* col, float* scale) {
    const int sz = NMT * NTV * 256;
    int d, rho;
    if (idx < sz) {
        const int r = idx & 3, lane = (idx >> 2) & 63, nt = (idx >> 8) % NTV;
        d = (idx >> 8) / NTV;
        rho = 4 * (lane >> 4) + r;
        *col = 16 * nt + (lane & 15);
    } else {
        const int e = idx - sz;
        d = e / 16;
        rho = e % 16;
        *col = -1;                                   // z entry
    }
    if (d == 8 && rho >= 8) return -1;
    const int i = rho, j = (rho + d) & 15;
    const int a = min(i, j), b = max(i, j);
    *scale = d == 0 ? 1.0f : kSqrt2;
    return a * DK - a * (a - 1) / 2 + (b - a);
}

__global__ void record_from_packed(float* __restrict__ rec, const float* __restrict__ S,
                                   const float* __restrict__ z, int NTV, int REC, int nrec) {
    const int D = DK * (DK + 1) / 2, DV = 16 * NTV;
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        const int idx = (int)(x % REC);
        int col;
        float scale;
        const int p = record_to_packed(idx, NTV, &col, &scale);
        float val = 0.0f;
        if (p >= 0) val = (col >= 0 ? S[(b * D + p) * DV + col] : z[b * D + p]) / scale;
        rec[x] = val;
    }
}

__global__ void record_to_packed_kernel(const float* __restrict__ rec, float* __restrict__ S,
                                        float* __restrict__ z, int NTV, int REC, int nrec) {
    const int D = DK * (DK + 1) / 2, DV = 16 * NTV;
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        const int idx = (int)(x % REC);
        int col;
        float scale;
        const int p = record_to_packed(idx, NTV, &col, &scale);
        if (p < 0) continue;
        const float val = rec[x] * scale;
        if (col >= 0) S[(b * D + p) * DV + col] = val;
        else z[b * D + p] = val;
    }
}

}  // namespace

hipError_t launch_record_from_packed16(float* rec, const float* S, const float* z, int dv,
                                       int nrec, hipStream_t st) {
    const int REC = mfma16_record_floats(dv);
    const size_t n = (size_t)REC * nrec;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    record_from_packed<<<blocks, 256, 0, st>>>(rec, S, z, dv / 16, REC, nrec);
    return hipGetLastError();
}

hipError_t launch_record_to_packed16(const float* rec, float* S, float* z, int dv, int nrec,
                                     hipStream_t st) {
    const int REC = mfma16_record_floats(dv);
    const size_t n = (size_t)REC * nrec;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    record_to_packed_kernel<<<blocks, 256, 0, st>>>(rec, S, z, dv / 16, REC, nrec);
    return hipGetLastError();
}

}  // namespace kata
