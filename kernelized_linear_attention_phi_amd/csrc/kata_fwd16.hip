// Fused bf16 chunked-state forward for d_k = 16 on gfx950 matrix cores.
//
// Method (KATA explainers, gist.science, technical summary 2.3; the paper's
// abstract): the sequence is cut into chunks of C positions; each output is the
// masked intra-chunk term plus phi(Q_c) times the prefix of chunk states; the
// prefix is propagated by an associative scan. Here one workgroup of two
// wavefronts owns a segment of G consecutive chunks of one (batch, head) and
// carries the running state S = sum phi(k) v^T across the segment in matrix-core
// accumulators, so only one state per segment touches HBM:
//   kata_seg_state16 : segment totals         (phi(K)^T V on MFMA)
//   (scan kernel)    : exclusive prefix over segments of each head
//   kata_fwd16       : per chunk, inter (phi(Q).S) and intra (QK^T -> square ->
//                      mask -> A.V) on MFMA, normalise, store, then
//                      S += phi(K)^T V.
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
// Work split inside a segment. Wavefront 0 owns feature tiles 0..3, wavefront 1
// tiles 4..7, and tile 8 is split by value tiles (the first half of them to
// wavefront 0): each lifts keys and queries for its own tiles only, updates its
// own rows of S, and computes partial numerators phi(Q).S for all query rows of
// the chunk over its own tiles. The partials for the other wavefront's query
// tiles (16-row tiles alternate between the two) go through LDS once per chunk;
// each wavefront then finishes its own query tiles (intra term, denominators,
// division). Wavefront 0 issues all chunk loads and no stores, wavefront 1 all
// output stores, so waiting for chunk data never waits for stores.
//
// Denominators. Inside a chunk, sum_j A_tj comes from the same MFMAs as the
// numerators through a value tile whose first column is 1 (the "ones" tile).
// Across chunks, z = sum phi(k) is kept as the 16 x 16 Gram matrix
// Z = sum k k^T (one accumulator tile; z is its packed upper triangle), and
// phi(q).z = q^T Z q is one MFMA (Z q) plus a 4-term dot product per lane.
#include "kata_chunk.h"
#include "kata_internal.h"
#include "kata_records.h"

#include <algorithm>

namespace kata {

namespace {

constexpr int DK = 16;
constexpr int NMT = 9;                  // feature tiles (delta = 0..8)
constexpr int NW = 2;                   // wavefronts per segment

template <int DV, int C>
struct Cfg {
    static constexpr int NTV = DV / 16;           // value tiles
    static constexpr int TT = C / 16;             // query tiles per chunk
    static constexpr int TW = TT / NW;            // query tiles per wavefront
    static constexpr int KS = C / 32;             // 32-token K-steps per chunk
    static constexpr int QB = C * DK * 2;         // bytes of a q or k chunk
    static constexpr int VB = C * DV * 2;         // bytes of a v chunk
    static constexpr int BUF = 2 * QB + VB;       // one chunk buffer
    static constexpr int NBUF = 2;                // staging depth (prefetch distance 1)
    static constexpr int XB = NW * TW * NTV * 1024;   // exchange of partial numerators
    static constexpr int OROW = DV * 2 + 16;      // LDS row stride of a staged output tile
    static constexpr int REC = NMT * NTV * 256 + 256;   // floats per state record
    static constexpr int H8 = (NTV + 1) / 2;      // value tiles of tile 8 held by wavefront 0
    static_assert(TW * 16 * OROW <= TW * NTV * 1024, "staged output fits its exchange half");
};

// Value tiles [lo8, hi8) of feature tile 8 belong to wavefront W.
template <int W, int NTV> __host__ __device__ constexpr int lo8() { return W == 0 ? 0 : (NTV + 1) / 2; }
template <int W, int NTV> __host__ __device__ constexpr int hi8() { return W == 0 ? (NTV + 1) / 2 : NTV; }

// Running state of wavefront W: feature tiles 4W..4W+3 of S for every value
// tile, value tiles [lo8, hi8) of tile 8, and the Gram matrix Z = sum k k^T
// (lane = column, rows 4g + r).
template <int DV, int C>
struct State {
    f32x4_t s[4][Cfg<DV, C>::NTV];
    f32x4_t x[Cfg<DV, C>::H8];
    f32x4_t zm;
};

// ---- per-chunk fragments ----------------------------------------------------

// V^T fragments of K-step m (slot s = token 32m + 16(s/4) + 4g + s%4, lane =
// value column), read transposed from the row-major chunk in LDS.
template <int DV, int C>
__device__ __forceinline__ void v_fragment_step(const bf16_t* bv, u32x4_t (&vop)[Cfg<DV, C>::NTV],
                                                int m, const Lane& L) {
#pragma unroll
    for (int nt = 0; nt < Cfg<DV, C>::NTV; ++nt) vop[nt] = v_fragment_tr<DV>(bv, m, nt, L);
}

// KT[jb][r] = k[16jb + 4g + r][c16] (fp32, exact) via an identity product.
template <int DV, int C>
__device__ __forceinline__ void k_transposed(const bf16_t* bk, f32x4_t (&KT)[Cfg<DV, C>::TT],
                                             const Lane& L) {
    using F = Cfg<DV, C>;
    const u32x2_t id = ident16(L);
#pragma unroll
    for (int jb = 0; jb < F::TT; ++jb) {
        const u32x2_t kf = lds_row<2 * DK, u32x2_t>(bk, 16 * jb + L.c16, 8 * L.g);
        KT[jb] = mma16(kf, id, zero4());
    }
}

// Lifted keys of feature tile D for the tokens of one K-step (slot s): lane c16
// holds row rho = c16, i.e. k_rho * k_{(rho+D) mod 16}; bf16 A operand.
template <int D>
__device__ __forceinline__ void lift_key_values(const float (&ka)[8], const Lane& L, float (&f)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        f[s] = ka[s] * partner<D>(ka[s]);
        if (D == 8 && L.c16 >= 8) f[s] = 0.0f;       // repeated pairs stay zero
    }
}

template <int D>
__device__ __forceinline__ u32x4_t lift_keys(const float (&ka)[8], const Lane& L) {
    float f[8];
    lift_key_values<D>(ka, L, f);
    return u32x4_t{pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7])};
}

// Lifted keys of own tile i of wavefront W (tiles 4W + i), in fp32.
template <int W>
__device__ __forceinline__ void lift_key_values_own(int i, const float (&ka)[8], const Lane& L,
                                                    float (&f)[8]) {
    switch (i) {
        case 0: return lift_key_values<4 * W + 0>(ka, L, f);
        case 1: return lift_key_values<4 * W + 1>(ka, L, f);
        case 2: return lift_key_values<4 * W + 2>(ka, L, f);
        default: return lift_key_values<4 * W + 3>(ka, L, f);
    }
}

// ---- decay gate --------------------------------------------------------------
// Per-token log-decays g <= 0 (state S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T, z
// likewise). Within a chunk, b_t = g_0 + ... + g_t (log2 units here); the
// inter-chunk term of query t decays by exp(b_t), key j inside the chunk by
// exp(b_t - b_j), and the state leaves the chunk scaled by exp(b_last) with key
// j weighted exp(b_last - b_j) (applied as sqrt to the key before the
// quadratic lift).

// State leaving a chunk: every accumulator scaled by a = exp(b_last) (the keys
// of the chunk are scaled inside state_update).
template <int DV, int C>
__device__ __forceinline__ void decay_state(State<DV, C>& st, const ChunkDecay& cd) {
    using F = Cfg<DV, C>;
    const float a = exp2_neg(cd.last);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) st.s[i][nt] *= a;
#pragma unroll
    for (int j = 0; j < F::H8; ++j) st.x[j] *= a;
    st.zm *= a;
}

// S(own tiles) += phi(K_c)^T V_c; Z += K_c^T K_c when WITH_Z. vop[m] are the V^T
// fragments. With the decay gate (DECAY), key j is first scaled by
// exp((b_last - b_j) / 2), i.e. its lift by exp(b_last - b_j). PREC takes the
// lifted keys as split operands (hi + lo, exact for unscaled bf16 keys), and the
// Gram product of scaled keys as hi*hi + hi*lo + lo*hi, so the state carries
// fp32-accurate sums.
template <int W, bool WITH_Z, int DV, int C, bool DECAY = false, bool PREC = false>
__device__ __forceinline__ void state_update(State<DV, C>& st, const f32x4_t (&KT)[Cfg<DV, C>::TT],
                                             const u32x4_t (&vop)[Cfg<DV, C>::KS][Cfg<DV, C>::NTV],
                                             const Lane& L,
                                             const KeyDecay& kd = KeyDecay{}) {
    using F = Cfg<DV, C>;
    constexpr int l8 = lo8<W, F::NTV>(), h8 = hi8<W, F::NTV>();
#pragma unroll
    for (int m = 0; m < F::KS; ++m) {
        float ka[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) ka[s] = KT[2 * m + s / 4][s % 4];
        if constexpr (DECAY) {
#pragma unroll
            for (int s = 0; s < 8; ++s)
                ka[s] *= exp2_neg(0.5f * (kd.last - kd.b(2 * m + s / 4, s % 4)));
        }
        if constexpr (WITH_Z) {
            // Gram matrix: A = K^T (row = coordinate c16), B = K (column = c16);
            // unscaled bf16 keys are exact operands
            if constexpr (PREC && DECAY) {
                u32x4_t kh, kl;
                split8(ka, kh, kl);
                st.zm = mma32(kh, kh, st.zm);
                st.zm = mma32(kh, kl, st.zm);
                st.zm = mma32(kl, kh, st.zm);
            } else {
                const u32x4_t kt = {pk2(ka[0], ka[1]), pk2(ka[2], ka[3]), pk2(ka[4], ka[5]), pk2(ka[6], ka[7])};
                st.zm = mma32(kt, kt, st.zm);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float f[8];
            lift_key_values_own<W>(i, ka, L, f);
            if constexpr (PREC) {
                u32x4_t fh, fl;
                split8(f, fh, fl);
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) {
                    st.s[i][nt] = mma32(fh, vop[m][nt], st.s[i][nt]);
                    st.s[i][nt] = mma32(fl, vop[m][nt], st.s[i][nt]);
                }
            } else {
                const u32x4_t fk = {pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7])};
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) st.s[i][nt] = mma32(fk, vop[m][nt], st.s[i][nt]);
            }
        }
        if constexpr (h8 > l8) {
            float f[8];
            lift_key_values<8>(ka, L, f);
            if constexpr (PREC) {
                u32x4_t fh, fl;
                split8(f, fh, fl);
#pragma unroll
                for (int j = 0; j < h8 - l8; ++j) {
                    st.x[j] = mma32(fh, vop[m][l8 + j], st.x[j]);
                    st.x[j] = mma32(fl, vop[m][l8 + j], st.x[j]);
                }
            } else {
                const u32x4_t fk = {pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7])};
#pragma unroll
                for (int j = 0; j < h8 - l8; ++j) st.x[j] = mma32(fk, vop[m][l8 + j], st.x[j]);
            }
        }
    }
}

// Lifted queries (x2 off the diagonal) of tiles (d0, d1) as a B operand: slot
// s = 4h + r is tile d_h, row rho = 4g + r, i.e. q_rho * q_{rho + d_h}; qr is
// q rotated by 4g (qr[x] = q[(x + 4g) mod 16]).
__device__ __forceinline__ void lift_query_values(const float (&qr)[16], int d0, int d1,
                                                  float (&f)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int d = h ? d1 : d0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            f[4 * h + r] = d == 0 ? qr[r] * qr[r] : (2.0f * qr[r]) * qr[(r + d) & 15];
    }
}

__device__ __forceinline__ u32x4_t lift_queries(const float (&qr)[16], int d0, int d1) {
    float f[8];
    lift_query_values(qr, d0, d1, f);
    return u32x4_t{pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7])};
}

// q row t = 16 tt + c16 of the staged chunk, rotated by 4g lanes; qf = q_t[4g..4g+3].
__device__ __forceinline__ void load_query(const bf16_t* bq, int tt, const Lane& L, float (&qr)[16],
                                           u32x2_t& qf) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const u32x2_t piece = lds_row<2 * DK, u32x2_t>(bq, 16 * tt + L.c16, 8 * ((L.g + a) & 3));
        if (a == 0) qf = piece;
        qr[4 * a + 0] = lo_bf16(piece[0]);
        qr[4 * a + 1] = hi_bf16(piece[0]);
        qr[4 * a + 2] = lo_bf16(piece[1]);
        qr[4 * a + 3] = hi_bf16(piece[1]);
    }
}

// ---- state records -----------------------------------------------------------
// A record holds one state in accumulator order: S at
// ((tile * NTV + nt) * 64 + lane) * 4 + r, then Z at NMT*NTV*256 + lane*4 + r.

template <int W, bool WITH_Z, int DV, int C>
__device__ __forceinline__ void record_store(float* rec, const State<DV, C>& st, const Lane& L) {
    using F = Cfg<DV, C>;
    constexpr int l8 = lo8<W, F::NTV>(), h8 = hi8<W, F::NTV>();
    f32x4_t* r4 = reinterpret_cast<f32x4_t*>(rec);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt)
            r4[((4 * W + i) * F::NTV + nt) * 64 + L.lane] = st.s[i][nt];
#pragma unroll
    for (int j = 0; j < h8 - l8; ++j) r4[(8 * F::NTV + l8 + j) * 64 + L.lane] = st.x[j];
    if (WITH_Z) r4[NMT * F::NTV * 64 + L.lane] = st.zm;
}

template <int W, int DV, int C>
__device__ __forceinline__ void record_load(const float* rec, State<DV, C>& st, const Lane& L) {
    using F = Cfg<DV, C>;
    constexpr int l8 = lo8<W, F::NTV>(), h8 = hi8<W, F::NTV>();
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(rec);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt)
            st.s[i][nt] = r4[((4 * W + i) * F::NTV + nt) * 64 + L.lane];
#pragma unroll
    for (int j = 0; j < F::H8; ++j)
        st.x[j] = j < h8 - l8 ? r4[(8 * F::NTV + l8 + j) * 64 + L.lane] : zero4();
    st.zm = r4[NMT * F::NTV * 64 + L.lane];
}

// ---- per-wavefront bodies --------------------------------------------------------

template <int W, int DV, int C, bool DECAY, bool PREC>
__device__ __forceinline__ void seg_state_body(const bf16_t* k, const bf16_t* v, const float* gdec,
                                               float* rec, float* segdec, char* lds, int T,
                                               int NC, int G, int NSEG, const Lane& L) {
    using F = Cfg<DV, C>;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    LoadPipeline<DK, DV, C, NW, 3, DECAY> P{lds, seg * G, min(NC, seg * G + G), T, bh * T, gdec};
    float lsum = 0.0f;                             // log2 of the segment's decay
    State<DV, C> st;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) st.s[i][nt] = zero4();
#pragma unroll
    for (int j = 0; j < F::H8; ++j) st.x[j] = zero4();
    st.zm = zero4();

    P.prologue(k, v, L);
    for (int c = P.c0; c < P.c1; ++c) {
        P.acquire(k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::QB);
        f32x4_t KT[F::TT];
        k_transposed<DV, C>(bk, KT, L);
        KeyDecay kd{};
        if constexpr (DECAY) {
            const ChunkDecay cd = chunk_decay<C>(buf + 2 * F::QB + F::VB, L);
            kd = key_decays(cd, reinterpret_cast<float*>(lds + 3 * ChunkIO<DK, DV, C, NW, NW, DECAY>::BUF +
                                                          W * kKeyDecayRowBytes), L);
            decay_state<DV, C>(st, cd);
            lsum += cd.last;
        }
        u32x4_t vop[F::KS][F::NTV];
#pragma unroll
        for (int m = 0; m < F::KS; ++m) v_fragment_step<DV, C>(bv, vop[m], m, L);
        // the Gram matrix goes with wavefront 1 (wavefront 0 holds more of tile 8
        // when the value tiles are odd)
        state_update<W, W == 1, DV, C, DECAY, PREC>(st, KT, vop, L, kd);
        compiler_fence();
    }
    record_store<W, W == 1, DV, C>(rec + (bh * NSEG + seg) * (size_t)F::REC, st, L);
    if (DECAY && W == 0 && L.lane == 0) segdec[bh * NSEG + seg] = exp2_neg(lsum);
}

// Stores the output rows one wavefront staged in LDS (its exchange half, row
// stride OROW, query tiles NW*u + w): row r of the staged tiles goes to
// oc[16*NW*(r/16) + r%16] if that is below n (the caller offsets oc and n by the
// 16 w rows of the staging wavefront); issued by wavefront 1 only.
template <int DV, int C>
__device__ __forceinline__ void store_staged_rows(const char* ostage, bf16_t* oc, int n,
                                                  const Lane& L) {
    using F = Cfg<DV, C>;
    constexpr int UPR = DV * 2 / 16;              // 16-byte units per row
    constexpr int NU = F::TW * 16 * UPR;
#pragma unroll
    for (int i = 0; i < (NU + 63) / 64; ++i) {
        const int unit = L.lane + 64 * i;
        if (unit < NU) {
            const int rl = unit / UPR, col = unit % UPR;
            const int row = 16 * NW * (rl / 16) + rl % 16;
            const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ostage + rl * F::OROW + 16 * col);
            if (row < n) *reinterpret_cast<u32x4_t*>(oc + (size_t)row * DV + 8 * col) = val;
        }
    }
}

// Memory roles: wavefront 0 issues every direct-to-LDS load and no global store,
// so its wait for chunk data never waits for stores; wavefront 1 issues every
// output store and never waits for them. Both stage their output rows in LDS
// (their own exchange half); wavefront 1 stores its rows in the same chunk and
// wavefront 0's one chunk later, as whole rows.
template <int W, int DV, int C, bool CAUSAL, bool DECAY, bool PREC>
__device__ __forceinline__ void fwd_body(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                         const float* gdec, const float* prefix,
                                         float* final_rec, bf16_t* o, char* lds, int T, int NC,
                                         int G, int NSEG, const Lane& L) {
    using F = Cfg<DV, C>;
    using IO = ChunkIO<DK, DV, C, NW, 1, DECAY>;
    constexpr int l8 = lo8<W, F::NTV>(), h8 = hi8<W, F::NTV>();
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    Pipeline<DK, DV, C, NW, 1, DECAY> P{lds, seg * G, min(NC, seg * G + G), T, bh * T, true, gdec};
    // exchange buffer: partials for query tile (u of wavefront w) at [w][u][nt][lane];
    // half 0 then holds wavefront 0's staged output rows until the next chunk
    f32x4_t* xbuf = reinterpret_cast<f32x4_t*>(lds + F::NBUF * IO::BUF);
    char* ostage = reinterpret_cast<char*>(xbuf);

    State<DV, C> st;
    record_load<W, DV, C>(prefix + (CAUSAL ? bh * NSEG + seg : bh) * (size_t)F::REC, st, L);

    P.stage(q, k, v, P.c0, L);
    for (int c = P.c0; c < P.c1; ++c) {
        const int n = min(C, T - c * C);
        P.acquire_q(q, k, v, c, L);                   // q of chunk c visible
        const char* buf = P.buffer(c);
        const bf16_t* bq = reinterpret_cast<const bf16_t*>(buf);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::QB);
        bf16_t* oc = o + (bh * T + (size_t)c * C) * DV;

        // wavefront 0's rows of the previous chunk, before its half is reused
        if (W == 1 && c > P.c0) store_staged_rows<DV, C>(ostage, oc - (size_t)C * DV, C, L);
        compiler_fence();

        // ---- inter-chunk partials over this wavefront's feature tiles, for every
        // query tile; those of the other wavefront's tiles go to the exchange
        f32x4_t num[F::TW][F::NTV + 1];            // own query tiles (+ ones tile)
        if constexpr (PREC) {
            // Split operands: hi*hi + lo*hi + hi*lo per pair (the lifted query is
            // exact as hi + lo). Query tiles go in groups of two with the pair
            // loop inside, so one pair's split state operands and two tiles'
            // accumulators are live at a time.
            constexpr int TG = F::TT < 2 ? F::TT : 2;
#pragma unroll
            for (int t0 = 0; t0 < F::TT; t0 += TG) {
                f32x4_t acc[TG][F::NTV];
#pragma unroll
                for (int j = 0; j < TG; ++j)
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) acc[j][nt] = zero4();
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    u32x4_t sh[F::NTV], sl[F::NTV];
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) {
                        const f32x4_t& x = st.s[2 * p][nt];
                        const f32x4_t& y = st.s[2 * p + 1][nt];
                        sh[nt] = u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(y[0], y[1]), pk2(y[2], y[3])};
                        const u32x2_t a = lo_of(x, sh[nt][0], sh[nt][1]), b = lo_of(y, sh[nt][2], sh[nt][3]);
                        sl[nt] = u32x4_t{a[0], a[1], b[0], b[1]};
                    }
#pragma unroll
                    for (int j = 0; j < TG; ++j) {
                        float qr[16];
                        u32x2_t qf;
                        load_query(bq, t0 + j, L, qr, qf);
                        float f[8];
                        lift_query_values(qr, 4 * W + 2 * p, 4 * W + 2 * p + 1, f);
                        u32x4_t fh, fl;
                        split8(f, fh, fl);
#pragma unroll
                        for (int nt = 0; nt < F::NTV; ++nt) {
                            acc[j][nt] = mma32(sh[nt], fh, acc[j][nt]);
                            acc[j][nt] = mma32(sl[nt], fh, acc[j][nt]);
                            acc[j][nt] = mma32(sh[nt], fl, acc[j][nt]);
                        }
                    }
                }
                if constexpr (h8 > l8) {              // own value tiles of tile 8 (half K-step)
                    u32x2_t sh8[F::H8], sl8[F::H8];
#pragma unroll
                    for (int i = 0; i < h8 - l8; ++i) {
                        sh8[i] = u32x2_t{pk2(st.x[i][0], st.x[i][1]), pk2(st.x[i][2], st.x[i][3])};
                        sl8[i] = lo_of(st.x[i], sh8[i][0], sh8[i][1]);
                    }
#pragma unroll
                    for (int j = 0; j < TG; ++j) {
                        float qr[16];
                        u32x2_t qf;
                        load_query(bq, t0 + j, L, qr, qf);
                        float f[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) f[r] = (2.0f * qr[r]) * qr[(r + 8) & 15];
                        u32x2_t fh, fl;
                        split4(f, fh, fl);
#pragma unroll
                        for (int i = 0; i < h8 - l8; ++i) {
                            acc[j][l8 + i] = mma16_acc32(sh8[i], fh, acc[j][l8 + i]);
                            acc[j][l8 + i] = mma16_acc32(sl8[i], fh, acc[j][l8 + i]);
                            acc[j][l8 + i] = mma16_acc32(sh8[i], fl, acc[j][l8 + i]);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < TG; ++j) {
                    const int tt = t0 + j, u = tt / NW;
                    if (tt % NW == W) {
#pragma unroll
                        for (int nt = 0; nt < F::NTV; ++nt) num[u][nt] = acc[j][nt];
                        num[u][F::NTV] = zero4();
                    } else {
#pragma unroll
                        for (int nt = 0; nt < F::NTV; ++nt)
                            xbuf[((1 - W) * F::TW + u) * F::NTV * 64 + nt * 64 + L.lane] = acc[j][nt];
                    }
                }
            }
        } else {
            // S^T in bf16 as A operands: slot s of pair p = own tile 2p + s/4, row 4g + s%4
            u32x4_t sop[2][F::NTV];
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt)
                    sop[p][nt] = u32x4_t{pk2(st.s[2 * p][nt][0], st.s[2 * p][nt][1]),
                                         pk2(st.s[2 * p][nt][2], st.s[2 * p][nt][3]),
                                         pk2(st.s[2 * p + 1][nt][0], st.s[2 * p + 1][nt][1]),
                                         pk2(st.s[2 * p + 1][nt][2], st.s[2 * p + 1][nt][3])};
            u32x2_t sop8[F::H8];
#pragma unroll
            for (int j = 0; j < h8 - l8; ++j)
                sop8[j] = u32x2_t{pk2(st.x[j][0], st.x[j][1]), pk2(st.x[j][2], st.x[j][3])};
#pragma unroll
            for (int tt = 0; tt < F::TT; ++tt) {
                float qr[16];
                u32x2_t qf;
                load_query(bq, tt, L, qr, qf);
                f32x4_t part[F::NTV];
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) part[nt] = zero4();
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const u32x4_t fq = lift_queries(qr, 4 * W + 2 * p, 4 * W + 2 * p + 1);
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) part[nt] = mma32(sop[p][nt], fq, part[nt]);
                }
                if constexpr (h8 > l8) {              // own value tiles of tile 8 (half K-step)
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) f[r] = (2.0f * qr[r]) * qr[(r + 8) & 15];
                    const u32x2_t fq = {pk2(f[0], f[1]), pk2(f[2], f[3])};
#pragma unroll
                    for (int j = 0; j < h8 - l8; ++j)
                        part[l8 + j] = mma16_acc32(sop8[j], fq, part[l8 + j]);
                }
                const int u = tt / NW;
                if (tt % NW == W) {
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) num[u][nt] = part[nt];
                    num[u][F::NTV] = zero4();
                } else {
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt)
                        xbuf[((1 - W) * F::TW + u) * F::NTV * 64 + nt * 64 + L.lane] = part[nt];
                }
            }
        }
        P.wait_kv(c, L);                              // k, v of chunk c landed
        lds_barrier();                                // partials exchanged, k and v visible
#pragma unroll
        for (int u = 0; u < F::TW; ++u)
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt)
                num[u][nt] += xbuf[(W * F::TW + u) * F::NTV * 64 + nt * 64 + L.lane];
        // decay gate: the chunk's cumulative log-decays (staged with q, valid for
        // the whole chunk), computed here so that they are not live during the
        // inter-chunk products
        ChunkDecay cd{0.0f, 0.0f};
        KeyDecay kd{};
        float bq_own[F::TW];                        // b of this lane's query in own tile u
        if constexpr (DECAY) {
            cd = chunk_decay<C>(buf + 2 * F::QB + F::VB, L);
            kd = key_decays(cd, reinterpret_cast<float*>(lds + F::NBUF * IO::BUF + F::XB +
                                                          W * kKeyDecayRowBytes), L);
#pragma unroll
            for (int u = 0; u < F::TW; ++u) bq_own[u] = __shfl(cd.b, 16 * (NW * u + W) + L.c16, 64);
        }
        if constexpr (DECAY) {                        // the prefix state decays to query t
#pragma unroll
            for (int u = 0; u < F::TW; ++u) {
                const float e = exp2_neg(bq_own[u]);
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) num[u][nt] *= e;
            }
        }
        compiler_fence();                             // partials read before rows are staged

        // V^T fragments (intra term and state update; the split-operand variant
        // reads them where they are used rather than keep them live)
        u32x4_t vop[F::KS][F::NTV];
        if (CAUSAL && !PREC) {
#pragma unroll
            for (int m = 0; m < F::KS; ++m) v_fragment_step<DV, C>(bv, vop[m], m, L);
        }
        // Z as an A operand: lane c16 = row i, slots 4g + s = column j; Z is
        // symmetric, so the accumulator (lane = column) serves directly.
        const u32x2_t zop = {pk2(st.zm[0], st.zm[1]), pk2(st.zm[2], st.zm[3])};
        const u32x2_t zol = PREC ? lo_of(st.zm, zop[0], zop[1]) : u32x2_t{0u, 0u};
#pragma unroll
        for (int u = 0; u < F::TW; ++u) {
            const int tt = NW * u + W;
            const int t = 16 * tt + L.c16;
            float qr[16];
            u32x2_t qf;
            load_query(bq, tt, L, qr, qf);
            // ---- intra-chunk term: A = (Q K^T)^2 masked to j <= t, num += A [V | 1]
            if (CAUSAL) {
                const u32x4_t ones = ones_op(L);
#pragma unroll
                for (int m = 0; m <= tt / 2; ++m) {
                    const bool diag = 32 * m + 31 > 16 * tt;
                    float w[8];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x2_t kf =
                            lds_row<2 * DK, u32x2_t>(bk, 32 * m + 16 * h + L.c16, 8 * L.g);
                        // rows j = 32m + 16h + 4g + r, column t
                        const f32x4_t sc = mma16(kf, qf, zero4());
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = 32 * m + 16 * h + 4 * L.g + r;
                            float x = sc[r] * sc[r];
                            if constexpr (DECAY) x *= exp2_neg(bq_own[u] - kd.b(2 * m + h, r));
                            w[4 * h + r] = (!diag || j <= t) ? x : 0.0f;
                        }
                    }
                    const u32x4_t at = {pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]), pk2(w[6], w[7])};
                    if constexpr (PREC) {
#pragma unroll
                        for (int nt = 0; nt < F::NTV; ++nt)
                            num[u][nt] = mma32(v_fragment_tr<DV>(bv, m, nt, L), at, num[u][nt]);
                    } else {
#pragma unroll
                        for (int nt = 0; nt < F::NTV; ++nt) num[u][nt] = mma32(vop[m][nt], at, num[u][nt]);
                    }
                    num[u][F::NTV] = mma32(ones, at, num[u][F::NTV]);
                }
            }
            // ---- normalise: o = num / den
            // inter-chunk denominator q^T Z q: (Z q)[4g + r] times q[4g + r],
            // summed over r here and over the four lane groups below
            f32x4_t zq = mma16(zop, qf, zero4());
            if constexpr (PREC) zq = mma16(zol, qf, zq);   // q is exact in bf16
            float di = qr[0] * zq[0];
            di = __builtin_fmaf(qr[1], zq[1], di);
            di = __builtin_fmaf(qr[2], zq[2], di);
            di = __builtin_fmaf(qr[3], zq[3], di);
            di += __shfl_xor(di, 16, 64);
            di += __shfl_xor(di, 32, 64);
            if constexpr (DECAY) di *= exp2_neg(bq_own[u]);
            // intra-chunk denominator: row 0 of the ones tile (lane group 0)
            const float den = __shfl(num[u][F::NTV][0], L.c16, 64) + di;
            const float y = inv_den(den);                  // y = 0 gives o = 0
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt) {
                float ov[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ov[r] = num[u][nt][r] * y;
                }
                // staged in this wavefront's exchange half (its partials are consumed)
                *reinterpret_cast<u32x2_t*>(ostage + W * (F::XB / 2) + (16 * u + L.c16) * F::OROW +
                                            2 * (16 * nt + 4 * L.g)) = {pk2(ov[0], ov[1]),
                                                                        pk2(ov[2], ov[3])};
            }
        }
        // wavefront 1's own rows leave as whole 128-byte rows, read back from its
        // half before the next chunk's partials overwrite it
        compiler_fence();
        if (W == 1) store_staged_rows<DV, C>(ostage + F::XB / 2, oc + 16 * DV, n - 16, L);

        // ---- running state: S += phi(K_c)^T V_c, Z += K_c^T K_c (not needed
        // after the segment's last chunk unless the final state is asked for)
        if (CAUSAL && (c + 1 < P.c1 || final_rec)) {
            f32x4_t KT[F::TT];
            k_transposed<DV, C>(bk, KT, L);
            if constexpr (DECAY) decay_state<DV, C>(st, cd);
            if constexpr (PREC) {
                u32x4_t vup[F::KS][F::NTV];
#pragma unroll
                for (int m = 0; m < F::KS; ++m) v_fragment_step<DV, C>(bv, vup[m], m, L);
                state_update<W, true, DV, C, DECAY, PREC>(st, KT, vup, L, kd);
            } else {
                state_update<W, true, DV, C, DECAY, PREC>(st, KT, vop, L, kd);
            }
        }
        compiler_fence();
    }
    // wavefront 0's rows of the last chunk
    lds_barrier();
    if (W == 1) {
        const int cl = P.c1 - 1;
        store_staged_rows<DV, C>(ostage, o + (bh * T + (size_t)cl * C) * DV, min(C, T - cl * C), L);
    }
    // running state after the segment's last chunk (one segment per head: the
    // final state), when asked for
    if (CAUSAL && final_rec) record_store<W, W == 1, DV, C>(final_rec + bh * (size_t)F::REC, st, L);
}

// ---- kernels -------------------------------------------------------------------

template <int DV, int C, bool DECAY, bool PREC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kata_seg_state16(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                      const float* __restrict__ gdec, float* __restrict__ rec,
                      float* __restrict__ segdec, int T, int NC, int G, int NSEG) {
    __shared__ __attribute__((aligned(16)))
    char lds[3 * ChunkIO<DK, DV, C, NW, NW, DECAY>::BUF + (DECAY ? NW * kKeyDecayRowBytes : 0)];
    const Lane L;
    if (L.w == 0) seg_state_body<0, DV, C, DECAY, PREC>(k, v, gdec, rec, segdec, lds, T, NC, G, NSEG, as_wave<0>(L));
    else seg_state_body<1, DV, C, DECAY, PREC>(k, v, gdec, rec, segdec, lds, T, NC, G, NSEG, as_wave<1>(L));
}

// The gated variant's larger chunk buffers allow three workgroups per compute
// unit, not four, so it may also use more than 256 registers per lane (it would
// otherwise spill loop-invariant addresses).
template <int DV, int C, bool CAUSAL, bool DECAY, bool PREC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(DECAY ? 1 : 2, 2)))
void kata_fwd16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, const float* __restrict__ gdec,
                const float* __restrict__ prefix, float* __restrict__ final_rec,
                bf16_t* __restrict__ o, int T, int NC, int G, int NSEG) {
    using F = Cfg<DV, C>;
    __shared__ __attribute__((aligned(16)))
    char lds[F::NBUF * ChunkIO<DK, DV, C, NW, 1, DECAY>::BUF + F::XB + (DECAY ? NW * kKeyDecayRowBytes : 0)];
    const Lane L;
    if (L.w == 0)
        fwd_body<0, DV, C, CAUSAL, DECAY, PREC>(q, k, v, gdec, prefix, final_rec, o, lds, T, NC, G, NSEG, as_wave<0>(L));
    else
        fwd_body<1, DV, C, CAUSAL, DECAY, PREC>(q, k, v, gdec, prefix, final_rec, o, lds, T, NC, G, NSEG, as_wave<1>(L));
}

// Launch arguments shared by every shape: gdec (log-decays, NULL = no gate;
// the gated forward is causal only), segdec (per-segment decays, state kernel).
struct Args {
    const void *q, *k, *v;
    const float* gdec;
    float* rec;            // state kernel: segment records; output kernel: final_rec
    float* segdec;
    const float* prefix;
    void* o;
    int causal, G, NSEG;
    bool state_only;
    bool prec;             // split operands (the gated kernels always take them)
};

template <int DV, int C>
hipError_t launch_dv_c(const Shape& s, const Args& a, hipStream_t st) {
    dim3 grid(a.NSEG, s.B * s.H);
    const bf16_t *q = (const bf16_t*)a.q, *k = (const bf16_t*)a.k, *v = (const bf16_t*)a.v;
    bf16_t* o = (bf16_t*)a.o;
    if (a.state_only) {
        if (a.gdec)
            kata_seg_state16<DV, C, true, true><<<grid, 64 * NW, 0, st>>>(k, v, a.gdec, a.rec, a.segdec,
                                                                           s.T, s.NC, a.G, a.NSEG);
        else if (a.prec)
            kata_seg_state16<DV, C, false, true><<<grid, 64 * NW, 0, st>>>(k, v, nullptr, a.rec, nullptr,
                                                                            s.T, s.NC, a.G, a.NSEG);
        else
            kata_seg_state16<DV, C, false, false><<<grid, 64 * NW, 0, st>>>(k, v, nullptr, a.rec, nullptr,
                                                                             s.T, s.NC, a.G, a.NSEG);
    } else if (a.gdec) {
        kata_fwd16<DV, C, true, true, true><<<grid, 64 * NW, 0, st>>>(q, k, v, a.gdec, a.prefix, a.rec, o,
                                                                       s.T, s.NC, a.G, a.NSEG);
    } else if (a.causal) {
        if (a.prec)
            kata_fwd16<DV, C, true, false, true><<<grid, 64 * NW, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                            a.rec, o, s.T, s.NC, a.G, a.NSEG);
        else
            kata_fwd16<DV, C, true, false, false><<<grid, 64 * NW, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                             a.rec, o, s.T, s.NC, a.G, a.NSEG);
    } else {
        if (a.prec)
            kata_fwd16<DV, C, false, false, true><<<grid, 64 * NW, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                             a.rec, o, s.T, s.NC, a.G, a.NSEG);
        else
            kata_fwd16<DV, C, false, false, false><<<grid, 64 * NW, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                              a.rec, o, s.T, s.NC, a.G, a.NSEG);
    }
    return hipGetLastError();
}

template <int C>
hipError_t launch_c(const Shape& s, const Args& a, hipStream_t st) {
    switch (s.dv) {
        case 16: return launch_dv_c<16, C>(s, a, st);
        case 32: return launch_dv_c<32, C>(s, a, st);
        case 64: return launch_dv_c<64, C>(s, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch(const Shape& s, const Args& a, hipStream_t st) {
    if (a.gdec && !a.state_only && !a.causal) return hipErrorInvalidValue;
    switch (s.C) {
        case 32: return launch_c<32>(s, a, st);
        case 64: return launch_c<64>(s, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma16_supported(const Shape& s) {
    return s.bf16 && s.dk == 16 && (s.C == 32 || s.C == 64) &&
           (s.dv == 16 || s.dv == 32 || s.dv == 64);
}

int mfma16_record_floats(int dv) { return NMT * (dv / 16) * 256 + 256; }

hipError_t launch_seg_state16(const Shape& s, const void* k, const void* v, float* rec, int G,
                              int NSEG, bool prec, hipStream_t st) {
    return dispatch(s, Args{nullptr, k, v, nullptr, rec, nullptr, nullptr, nullptr, 1, G, NSEG, true, prec}, st);
}

hipError_t launch_seg_state16_decay(const Shape& s, const void* k, const void* v,
                                    const float* gdec, float* rec, float* segdec, int G, int NSEG,
                                    hipStream_t st) {
    return dispatch(s, Args{nullptr, k, v, gdec, rec, segdec, nullptr, nullptr, 1, G, NSEG, true, true}, st);
}

hipError_t launch_fwd16(const Shape& s, const void* q, const void* k, const void* v,
                        const float* prefix, float* final_rec, void* o, int causal, int G,
                        int NSEG, bool prec, hipStream_t st) {
    return dispatch(s, Args{q, k, v, nullptr, final_rec, nullptr, prefix, o, causal, G, NSEG, false, prec}, st);
}

hipError_t launch_fwd16_decay(const Shape& s, const void* q, const void* k, const void* v,
                              const float* gdec, const float* prefix, float* final_rec, void* o,
                              int G, int NSEG, hipStream_t st) {
    return dispatch(s, Args{q, k, v, gdec, final_rec, nullptr, prefix, o, 1, G, NSEG, false, true}, st);
}

// ---- per-chunk exclusive prefixes (kata_scan_states) ---------------------------
// One workgroup per segment starts from the segment's exclusive prefix (a
// scanned segment record) and walks its chunks: it writes the running state -
// the exclusive prefix of chunk c - to the packed S_prefix[c], z_prefix[c],
// then adds chunk c with split key operands (exact for bf16 keys), so every
// prefix is an fp32-accurate sum. Wavefront 0 writes feature tiles 0..3 and its
// value tiles of tile 8, wavefront 1 tiles 4..7, the rest of tile 8 and the
// Gram matrix (as z). Lanes 16g .. 16g + 15 write 16 consecutive value
// columns of one packed row.

namespace {

template <int W, int DV, int C>
__device__ __forceinline__ void store_packed16(const State<DV, C>& st, float* Sp, float* zp,
                                               const Lane& L) {
    using F = Cfg<DV, C>;
    constexpr int l8 = lo8<W, F::NTV>(), h8 = hi8<W, F::NTV>();
    auto put = [&](int tile, int nt, const f32x4_t& x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int col;
            float scale;
            bool lower;
            const int p = rec16_to_packed(((tile * F::NTV + nt) * 64 + L.lane) * 4 + r, F::NTV,
                                          &col, &scale, &lower);
            if (p >= 0) Sp[p * DV + col] = x[r] * scale;
        }
    };
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) put(4 * W + i, nt, st.s[i][nt]);
#pragma unroll
    for (int j = 0; j < h8 - l8; ++j) put(8, l8 + j, st.x[j]);
    if constexpr (W == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int col;
            float scale;
            bool lower;
            const int p = rec16_to_packed(NMT * F::NTV * 256 + L.lane * 4 + r, F::NTV, &col, &scale,
                                          &lower);
            if (!lower) zp[p] = st.zm[r] * scale;
        }
    }
}

template <int W, int DV, int C>
__device__ __forceinline__ void prefix_body(const bf16_t* k, const bf16_t* v, const float* prefix,
                                            float* Sp, float* zp, char* lds, int T, int NC, int G,
                                            int NSEG, const Lane& L) {
    using F = Cfg<DV, C>;
    constexpr int D = DK * (DK + 1) / 2;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int c0 = seg * G, c1 = min(NC, seg * G + G);
    // only the chunks whose state is added are staged (the last chunk's
    // prefix is written from the state before it)
    LoadPipeline<DK, DV, C, NW, 3, false> P{lds, c0, c1 - 1, T, bh * T, nullptr};
    State<DV, C> st;
    record_load<W, DV, C>(prefix + (bh * NSEG + seg) * (size_t)F::REC, st, L);
    P.prologue(k, v, L);
    for (int c = c0; c < c1 - 1; ++c) {
        store_packed16<W, DV, C>(st, Sp + (bh * NC + c) * (size_t)(D * DV), zp + (bh * NC + c) * (size_t)D, L);
        P.acquire(k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::QB);
        f32x4_t KT[F::TT];
        k_transposed<DV, C>(bk, KT, L);
        u32x4_t vop[F::KS][F::NTV];
#pragma unroll
        for (int m = 0; m < F::KS; ++m) v_fragment_step<DV, C>(bv, vop[m], m, L);
        state_update<W, W == 1, DV, C, false, true>(st, KT, vop, L);
        compiler_fence();
    }
    store_packed16<W, DV, C>(st, Sp + (bh * NC + c1 - 1) * (size_t)(D * DV),
                             zp + (bh * NC + c1 - 1) * (size_t)D, L);
}

template <int DV, int C>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kata_prefix16(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                   const float* __restrict__ prefix, float* __restrict__ Sp,
                   float* __restrict__ zp, int T, int NC, int G, int NSEG) {
    __shared__ __attribute__((aligned(16))) char lds[3 * ChunkIO<DK, DV, C, NW, NW, false>::BUF];
    const Lane L;
    if (L.w == 0) prefix_body<0, DV, C>(k, v, prefix, Sp, zp, lds, T, NC, G, NSEG, as_wave<0>(L));
    else prefix_body<1, DV, C>(k, v, prefix, Sp, zp, lds, T, NC, G, NSEG, as_wave<1>(L));
}

template <int C>
hipError_t launch_prefix16_c(const Shape& s, const void* k, const void* v, const float* prefix,
                             float* Sp, float* zp, int G, int NSEG, hipStream_t st) {
    dim3 grid(NSEG, s.B * s.H);
    const bf16_t *kk = (const bf16_t*)k, *vv = (const bf16_t*)v;
    switch (s.dv) {
        case 16: kata_prefix16<16, C><<<grid, 64 * NW, 0, st>>>(kk, vv, prefix, Sp, zp, s.T, s.NC, G, NSEG); break;
        case 32: kata_prefix16<32, C><<<grid, 64 * NW, 0, st>>>(kk, vv, prefix, Sp, zp, s.T, s.NC, G, NSEG); break;
        case 64: kata_prefix16<64, C><<<grid, 64 * NW, 0, st>>>(kk, vv, prefix, Sp, zp, s.T, s.NC, G, NSEG); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefix16(const Shape& s, const void* k, const void* v, const float* prefix,
                           float* Sp, float* zp, int G, int NSEG, hipStream_t st) {
    switch (s.C) {
        case 32: return launch_prefix16_c<32>(s, k, v, prefix, Sp, zp, G, NSEG, st);
        case 64: return launch_prefix16_c<64>(s, k, v, prefix, Sp, zp, G, NSEG, st);
    }
    return hipErrorInvalidValue;
}

// ---- record <-> packed state conversion ------------------------------------

namespace {

__global__ void record_from_packed(float* __restrict__ rec, const float* __restrict__ S,
                                   const float* __restrict__ z, int NTV, int REC, int nrec) {
    const int D = DK * (DK + 1) / 2, DV = 16 * NTV;
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        const int idx = (int)(x % REC);
        int col;
        float scale;
        bool lower;
        const int p = rec16_to_packed(idx, NTV, &col, &scale, &lower);
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
        bool lower;
        const int p = rec16_to_packed(idx, NTV, &col, &scale, &lower);
        if (p < 0 || lower) continue;
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
