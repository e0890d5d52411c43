// Fused bf16 chunked-state forward for d_k = 32 on gfx950 matrix cores.
//
// Method (KATA explainers, gist.science, technical summary 2.3; the paper's
// abstract): the sequence is cut into chunks of C positions; each output is the
// masked intra-chunk term plus phi(Q_c) times the prefix of chunk states; the
// prefix is propagated by an associative scan. One workgroup (eight wavefronts
// at C = 128, four at C = 64) owns a segment of G consecutive chunks of one
// (batch, head) and carries the running state S = sum phi(k) v^T in registers
// across the segment:
//   kata_seg_state32 : segment totals         (phi(K)^T V on MFMA)
//   (scan kernel)    : exclusive prefix over segments of each head
//   kata_fwd32       : per chunk, inter (phi(Q).S) and intra (QK^T -> square ->
//                      mask -> A.V) on MFMA, normalise, store, then
//                      S += phi(K)^T V.
//
// Feature order. With L = coordinates 0..15 and U = 16..31 of a key, the
// D = 528 unique products x_a x_b fill exactly 33 tiles of 16 rows rho:
//   tiles  0..7  : L[rho] * L[(rho + delta) mod 16],  delta = 0..7
//   tiles  8..15 : U[rho] * U[(rho + delta) mod 16],  delta = 0..7
//   tiles 16..31 : L[rho] * U[(rho + delta) mod 16],  delta = 0..15
//   tile  32     : L[rho] * L[rho + 8] (rho < 8), U[rho - 8] * U[rho] (rho >= 8)
// so every key lift is a product of a lane's own coordinate with a DPP-rotated
// one, and no row is padding. The state holds plain sums of k_a k_b v; the
// factor 2 of an off-diagonal pair sits on the query side.
//
// Work split (NW wavefronts, TPW = 32 / NW). Wavefront w owns feature tiles
// TPW*w .. TPW*w + TPW - 1 for every value tile, one value tile of tile 32 (the
// last four wavefronts with eight, wavefront nt with four) and, for w < 4, one
// Gram tile (below): it lifts keys only for those and updates only those rows
// of S. Once per chunk each wavefront writes its part of S (as bf16
// matrix-core operands) to LDS; each wavefront then finishes its own query
// tiles against the whole state (tile w, and tile TT-1-w when it owns two), so
// the causal intra-chunk work is balanced and no partial sums are exchanged.
//
// Denominators. Inside a chunk, sum_j A_tj comes from the A.V MFMAs through a
// "ones" value tile. Across chunks, z = sum phi(k) is kept as the Gram matrix
// Z = sum k k^T in four 16 x 16 tiles (LL, LU, UL, UU; wavefront w keeps tile
// w), and phi(q).z = q^T Z q is two MFMAs (Z q) plus an 8-term dot product.
//
// Decay gate (DECAY, causal): the chunk's log-decays are staged after v; each
// wavefront keeps the cumulative values b of the chunk's positions in an LDS
// row of its own. Key coordinates are scaled by 2^{(b_last - b_j)/2} before the
// quadratic lift and the Gram product (so S and Z receive 2^{b_last - b_j}), the
// state by 2^{b_last} per chunk, the prefix term and q^T Z q of query t by
// 2^{b_t}, and the intra weights by 2^{b_t - b_j}.
#include "kata_chunk.h"
#include "kata_internal.h"
#include "kata_records.h"

#include <algorithm>
#include <type_traits>

namespace kata {

namespace {

constexpr int DK = 32;
constexpr int NFT = 33;                 // feature tiles
constexpr int NZ = 4;                   // Gram tiles

// Wavefronts per segment: eight (two per SIMD) when the chunk has eight query
// tiles, four otherwise.
template <int C> __host__ __device__ constexpr int nw32() { return C == 128 ? 8 : 4; }
template <int C> constexpr int kThreads32 = 64 * nw32<C>();
template <int C> constexpr int kWavesPerSimd32 = nw32<C>() / 4;

template <int DV, int C, bool GATE = false>
struct Cfg32 {
    static constexpr int NW = nw32<C>();
    static constexpr int TPW = 32 / NW;           // full feature tiles per wavefront
    static constexpr int NTV = DV / 16;           // value tiles
    static constexpr int TT = C / 16;             // query tiles per chunk
    static constexpr int TW = TT / NW;            // query tiles per wavefront
    static constexpr int KS = C / 32;             // 32-token K-steps per chunk
    using IO = ChunkIO<DK, DV, C, NW, NW, GATE>;
    // LDS (output kernel): bf16 state operands | two chunk buffers | one output
    // tile per wavefront
    static constexpr int SPAIR = 16 * NTV * 1024;   // S^T operands of tile pairs 0..15
    static constexpr int S32 = NTV * 512;           // S^T operands of tile 32
    static constexpr int ZOP = 2 * 1024;            // Gram operands (rows L, rows U)
    static constexpr int SB = SPAIR + S32 + ZOP;
    static constexpr int OROW = DV * 2 + 16;        // LDS row stride of a staged output tile
    static constexpr int OTILE = 16 * OROW;
    static constexpr int OU = 2 * DV;               // 16-byte units per 16-row output tile
    static constexpr int KROW = GATE ? 4 * C : 0;   // key-decay row of one wavefront
    static constexpr int LDS_FWD = 2 * IO::BUF + SB + NW * OTILE + NW * KROW;
    static constexpr int LDS_SEG = 4 * IO::BUF + NW * KROW;   // 4-deep staging of k | v (| g)
    static constexpr int REC = NFT * NTV * 256 + NZ * 256;   // floats per state record
    static_assert(TW >= 1, "at least one query tile per wavefront");
    static_assert(NW * TPW == 32 && TPW % 2 == 0, "tile pairs do not straddle wavefronts");
};

// Ownership. Wavefront W holds full tiles TPW*W .. TPW*W + TPW - 1 for every
// value tile; value tile xnt of tile 32 when has_x (the last four wavefronts
// with eight, wavefront nt with four); Gram tile W when W < 4.
template <int DV, int C, int W> __host__ __device__ constexpr bool has_x() {
    return Cfg32<DV, C>::NW == 8 ? (W >= 4 && W - 4 < Cfg32<DV, C>::NTV) : (W < Cfg32<DV, C>::NTV);
}
template <int DV, int C, int W> __host__ __device__ constexpr int xnt() {
    return Cfg32<DV, C>::NW == 8 ? W - 4 : W;
}
// feature class of tile t: 0 = L-circulant, 1 = U-circulant, 2 = cross
__host__ __device__ constexpr int tile_class(int t) { return t < 8 ? 0 : t < 16 ? 1 : 2; }
template <int DV, int C, int W> __host__ __device__ constexpr bool needs_l() {
    constexpr int t0 = Cfg32<DV, C>::TPW * W;
    return tile_class(t0) != 1 || has_x<DV, C, W>() || (W < 4 && W != 3);
}
template <int DV, int C, int W> __host__ __device__ constexpr bool needs_u() {
    constexpr int t0 = Cfg32<DV, C>::TPW * W;
    return tile_class(t0) != 0 || has_x<DV, C, W>() || (W >= 1 && W < 4);
}

// Running state of one wavefront (see the ownership rules above).
template <int DV, int C>
struct State32 {
    f32x4_t s[Cfg32<DV, C>::TPW][Cfg32<DV, C>::NTV];
    f32x4_t x;
    f32x4_t z;
};

// Query tile of slot u of wavefront W.
template <int W, int TT, int NW>
__device__ __forceinline__ constexpr int own_query_tile(int u) {
    return u == 0 ? W : TT - 1 - W;
}

// ---- lifts -----------------------------------------------------------------------

// phi(K) rows of feature tile T for the 8 tokens of one K-step: kl / ku hold
// coordinate c16 / 16 + c16 of each token (fp32, exact).
template <int T>
__device__ __forceinline__ void lift_key_values32(const float (&kl)[8], const float (&ku)[8],
                                                  float (&f)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if constexpr (T < 8) f[s] = kl[s] * partner<T>(kl[s]);
        else if constexpr (T < 16) f[s] = ku[s] * partner<T - 8>(ku[s]);
        else f[s] = kl[s] * partner<T - 16>(ku[s]);
    }
}

// Tile 32: rows < 8 pair L[rho] with L[rho + 8], rows >= 8 pair U[rho] with
// U[rho - 8]; b is chosen so that the rotated fetch lands on the right half.
__device__ __forceinline__ void lift_key_values_mixed(const float (&kl)[8], const float (&ku)[8],
                                                      const Lane& L, float (&f)[8]) {
    const bool lo = L.c16 < 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float a = lo ? kl[s] : ku[s];
        const float b = lo ? ku[s] : kl[s];
        f[s] = a * partner<8>(b);
    }
}

// Compile-time loop.
template <int P, int NP, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (P < NP) {
        f(std::integral_constant<int, P>{});
        static_for<P + 1, NP>(f);
    }
}

// One query row (t = 16 tt + c16) in registers: a[x] = q[(x + 4g) mod 16],
// b[x] = q[16 + (x + 4g) mod 16], a2 / b2 = 2 a / 2 b for x < 4, and the raw bf16
// q[4g..4g+3] | q[16+4g..16+4g+3] (the B operand of Z q).
struct QueryRow {
    float a[16], b[16], a2[4], b2[4];
    u32x4_t zf;
};

__device__ __forceinline__ void load_query32(const bf16_t* bq, int tt, const Lane& L, QueryRow& Q) {
    const int row = 16 * tt + L.c16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float* dst = h ? Q.b : Q.a;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x2_t piece = lds_row<2 * DK, u32x2_t>(bq, row, 32 * h + 8 * ((L.g + p) & 3));
            if (p == 0) {
                Q.zf[2 * h] = piece[0];
                Q.zf[2 * h + 1] = piece[1];
            }
            dst[4 * p + 0] = lo_bf16(piece[0]);
            dst[4 * p + 1] = hi_bf16(piece[0]);
            dst[4 * p + 2] = lo_bf16(piece[1]);
            dst[4 * p + 3] = hi_bf16(piece[1]);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        Q.a2[r] = 2.0f * Q.a[r];
        Q.b2[r] = 2.0f * Q.b[r];
    }
}

// phi(q) entry of feature tile T, row 4g + r (off-diagonal entries doubled).
template <int T>
__device__ __forceinline__ float query_entry(const QueryRow& Q, int r, bool lo_rows) {
    if constexpr (T == 0) return Q.a[r] * Q.a[r];
    else if constexpr (T < 8) return Q.a2[r] * Q.a[(r + T) & 15];
    else if constexpr (T == 8) return Q.b[r] * Q.b[r];
    else if constexpr (T < 16) return Q.b2[r] * Q.b[(r + T - 8) & 15];
    else if constexpr (T < 32) return Q.a2[r] * Q.b[(r + T - 16) & 15];
    else return lo_rows ? Q.a2[r] * Q.a[r + 8] : Q.b2[r] * Q.b[r + 8];
}

// The entries of the tile pair (T, T + 1) in B-operand slot order, in fp32.
template <int T>
__device__ __forceinline__ void query_pair_values(const QueryRow& Q, const Lane& L, float (&f)[8]) {
    const bool lo = L.g < 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f[r] = query_entry<T>(Q, r, lo);
        f[4 + r] = query_entry<T + 1>(Q, r, lo);
    }
}

// B operand of the tile pair (T, T + 1): slots 0..3 = tile T rows 4g + s,
// slots 4..7 = tile T + 1.
template <int T>
__device__ __forceinline__ u32x4_t lift_query_pair(const QueryRow& Q, const Lane& L) {
    const bool lo = L.g < 2;
    return u32x4_t{pk2(query_entry<T>(Q, 0, lo), query_entry<T>(Q, 1, lo)),
                   pk2(query_entry<T>(Q, 2, lo), query_entry<T>(Q, 3, lo)),
                   pk2(query_entry<T + 1>(Q, 0, lo), query_entry<T + 1>(Q, 1, lo)),
                   pk2(query_entry<T + 1>(Q, 2, lo), query_entry<T + 1>(Q, 3, lo))};
}

__device__ __forceinline__ u32x2_t lift_query_mixed(const QueryRow& Q, const Lane& L) {
    const bool lo = L.g < 2;
    return u32x2_t{pk2(query_entry<32>(Q, 0, lo), query_entry<32>(Q, 1, lo)),
                   pk2(query_entry<32>(Q, 2, lo), query_entry<32>(Q, 3, lo))};
}

// ---- K^T fragments ----------------------------------------------------------------

// kl[s] / ku[s] = k[token(s)][c16] / k[token(s)][16 + c16] for the 8 tokens of
// K-step m (slot s = token 32m + 16(s/4) + 4g + s%4), via identity products.
template <bool NEED_L, bool NEED_U>
__device__ __forceinline__ void key_columns(const bf16_t* bk, int m, const Lane& L,
                                            float (&kl)[8], float (&ku)[8]) {
    const u32x2_t id = ident16(L);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 32 * m + 16 * h + L.c16;
        f32x4_t tl = zero4(), tu = zero4();
        if constexpr (NEED_L) tl = mma16(lds_row<2 * DK, u32x2_t>(bk, row, 8 * L.g), id, zero4());
        if constexpr (NEED_U) tu = mma16(lds_row<2 * DK, u32x2_t>(bk, row, 32 + 8 * L.g), id, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            kl[4 * h + r] = tl[r];
            ku[4 * h + r] = tu[r];
        }
    }
}

__device__ __forceinline__ u32x4_t pack8(const float (&x)[8]) {
    return u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(x[4], x[5]), pk2(x[6], x[7])};
}

// S(own tiles) += phi(K_m)^T V_m, Z(own tile) += K_m^T K_m over one K-step;
// with DECAY each key weighted 2^{b_last - b_j}. PREC takes the lifted keys as
// split operands (hi + lo; exact for unscaled bf16 keys) and the Gram product of
// scaled keys as hi*hi + hi*lo + lo*hi, so the state carries fp32-accurate sums.
template <int W, int DV, int C, bool DECAY = false, bool PREC = false>
__device__ __forceinline__ void state_step(State32<DV, C>& st, const bf16_t* bk, const bf16_t* bv,
                                           int m, const Lane& L, const KeyDecay& kd = KeyDecay{}) {
    using F = Cfg32<DV, C>;
    float kl[8], ku[8];
    key_columns<needs_l<DV, C, W>(), needs_u<DV, C, W>()>(bk, m, L, kl, ku);
    if constexpr (DECAY) {
        // slot s is token 32m + 16(s/4) + 4g + s%4; both factors of every lifted
        // product and of the Gram product carry the square root of its weight
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float f = exp2_neg(0.5f * (kd.last - kd.b(2 * m + s / 4, s % 4)));
            kl[s] *= f;
            ku[s] *= f;
        }
    }
    if constexpr (W < 4) {
        // Gram tile W: LL, LU, UL, UU (A rows = first half, B columns = second)
        if constexpr (PREC && DECAY) {
            u32x4_t a, al, b, bl;
            split8(W < 2 ? kl : ku, a, al);
            split8(W == 0 || W == 2 ? kl : ku, b, bl);
            st.z = mma32(a, b, st.z);
            st.z = mma32(a, bl, st.z);
            st.z = mma32(al, b, st.z);
        } else {
            const u32x4_t gl = pack8(kl), gu = pack8(ku);
            if constexpr (W == 0) st.z = mma32(gl, gl, st.z);
            else if constexpr (W == 1) st.z = mma32(gl, gu, st.z);
            else if constexpr (W == 2) st.z = mma32(gu, gl, st.z);
            else st.z = mma32(gu, gu, st.z);
        }
    }
    u32x4_t vop[F::NTV];
#pragma unroll
    for (int nt = 0; nt < F::NTV; ++nt) vop[nt] = v_fragment_tr<DV>(bv, m, nt, L);
    static_for<0, F::TPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        float f[8];
        lift_key_values32<F::TPW * W + i>(kl, ku, f);
        if constexpr (PREC) {
            u32x4_t fh, fl;
            split8(f, fh, fl);
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt) {
                st.s[i][nt] = mma32(fh, vop[nt], st.s[i][nt]);
                st.s[i][nt] = mma32(fl, vop[nt], st.s[i][nt]);
            }
        } else {
            const u32x4_t fk = pack8(f);
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt) st.s[i][nt] = mma32(fk, vop[nt], st.s[i][nt]);
        }
    });
    if constexpr (has_x<DV, C, W>()) {
        float f[8];
        lift_key_values_mixed(kl, ku, L, f);
        if constexpr (PREC) {
            u32x4_t fh, fl;
            split8(f, fh, fl);
            st.x = mma32(fh, vop[xnt<DV, C, W>()], st.x);
            st.x = mma32(fl, vop[xnt<DV, C, W>()], st.x);
        } else {
            st.x = mma32(pack8(f), vop[xnt<DV, C, W>()], st.x);
        }
    }
}

// ---- decay gate ---------------------------------------------------------------------

// Cumulative log2-decays of the staged chunk written to this wavefront's row
// (position p at row[p], C = 128 takes positions lane and 64 + lane); returns
// the view of KeyDecay with last = b_{C-1}.
template <int C>
__device__ __forceinline__ KeyDecay chunk_key_decays(const char* staged_g, float* wrow,
                                                     const Lane& L) {
    if constexpr (C <= 64) {
        return key_decays(chunk_decay<C>(staged_g, L), wrow, L);
    } else {
        static_assert(C == 128, "chunk of 64 or 128 positions");
        const float* g = reinterpret_cast<const float*>(staged_g);
        float lo = g[L.lane] * kLog2e, hi = g[64 + L.lane] * kLog2e;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float ylo = __shfl_up(lo, d, 64);
            const float yhi = __shfl_up(hi, d, 64);
            if (L.lane >= d) {
                lo += ylo;
                hi += yhi;
            }
        }
        hi += __shfl(lo, 63, 64);
        wrow[L.lane] = lo;
        wrow[64 + L.lane] = hi;
        return KeyDecay{wrow + 4 * L.g, __shfl(hi, 63, 64)};
    }
}

// The running state leaving a chunk: every accumulator this wavefront holds
// times 2^{b_last}.
template <int W, int DV, int C>
__device__ __forceinline__ void decay_state32(State32<DV, C>& st, float last) {
    using F = Cfg32<DV, C>;
    const float a = exp2_neg(last);
#pragma unroll
    for (int i = 0; i < F::TPW; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) st.s[i][nt] *= a;
    if constexpr (has_x<DV, C, W>()) st.x *= a;
    if constexpr (W < 4) st.z *= a;
}

// ---- state records: S unit (tile t, value tile nt) at ((t*NTV + nt)*64 + lane)*4 + r,
// Gram tile zt at NFT*NTV*256 + (zt*64 + lane)*4 + r -----------------------------------

template <int W, int DV, int C>
__device__ __forceinline__ void record_store32(float* rec, const State32<DV, C>& st, const Lane& L) {
    using F = Cfg32<DV, C>;
    f32x4_t* r4 = reinterpret_cast<f32x4_t*>(rec);
#pragma unroll
    for (int i = 0; i < F::TPW; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt)
            r4[((F::TPW * W + i) * F::NTV + nt) * 64 + L.lane] = st.s[i][nt];
    if constexpr (has_x<DV, C, W>()) r4[(32 * F::NTV + xnt<DV, C, W>()) * 64 + L.lane] = st.x;
    if constexpr (W < 4) r4[(NFT * F::NTV + W) * 64 + L.lane] = st.z;
}

template <int W, int DV, int C>
__device__ __forceinline__ void record_load32(const float* rec, State32<DV, C>& st, const Lane& L) {
    using F = Cfg32<DV, C>;
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(rec);
#pragma unroll
    for (int i = 0; i < F::TPW; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt)
            st.s[i][nt] = r4[((F::TPW * W + i) * F::NTV + nt) * 64 + L.lane];
    st.x = has_x<DV, C, W>() ? r4[(32 * F::NTV + xnt<DV, C, W>()) * 64 + L.lane] : zero4();
    st.z = W < 4 ? r4[(NFT * F::NTV + W) * 64 + L.lane] : zero4();
}

// bf16 operands of this wavefront's part of the state, for every wavefront:
// pair p, value tile nt at SPAIR-offset ((p*NTV + nt)*64 + lane)*16 (A = S^T:
// lane = value column, slots 0..3 = tile 2p rows 4g+s, 4..7 = tile 2p+1);
// tile 32 at S32-offset (nt*64 + lane)*8; Gram rows L (Z_LL | Z_UL) and rows U
// (Z_LU | Z_UU) at ZOP-offset (half*64 + lane)*16 (+8 for the second tile).
template <int W, int DV, int C>
__device__ __forceinline__ void publish_state(char* sb, const State32<DV, C>& st, const Lane& L) {
    using F = Cfg32<DV, C>;
#pragma unroll
    for (int j = 0; j < F::TPW / 2; ++j)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) {
            const f32x4_t& x = st.s[2 * j][nt];
            const f32x4_t& y = st.s[2 * j + 1][nt];
            const int p = F::TPW / 2 * W + j;
            *reinterpret_cast<u32x4_t*>(sb + ((p * F::NTV + nt) * 64 + L.lane) * 16) =
                u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(y[0], y[1]), pk2(y[2], y[3])};
        }
    if constexpr (has_x<DV, C, W>())
        *reinterpret_cast<u32x2_t*>(sb + F::SPAIR + (xnt<DV, C, W>() * 64 + L.lane) * 8) =
            u32x2_t{pk2(st.x[0], st.x[1]), pk2(st.x[2], st.x[3])};
    if constexpr (W < 4) {
        constexpr int half = (W == 1 || W == 3) ? 1 : 0, part = W >= 2 ? 1 : 0;
        *reinterpret_cast<u32x2_t*>(sb + F::SPAIR + F::S32 + (half * 64 + L.lane) * 16 + part * 8) =
            u32x2_t{pk2(st.z[0], st.z[1]), pk2(st.z[2], st.z[3])};
    }
}

// ---- split-operand publication (PREC) ---------------------------------------------
// Split operands (hi + lo) double the published state, more than the LDS holds
// beside two chunk buffers, so it is published and consumed in two passes over
// half of the tile pairs each: pass 0 holds pairs 0..7 (wavefronts 0..NW/2-1),
// tile 32 and the Gram rows; pass 1 pairs 8..15 (the other wavefronts). Layout:
// hi of local pair pl, value tile nt at ((pl*NTV + nt)*64 + lane)*16, lo SPH
// bytes later; tile 32 hi / lo and Gram hi / lo after them, as in publish_state.
template <int DV, int C>
struct Prec32 {
    using F = Cfg32<DV, C>;
    static constexpr int SPH = 8 * F::NTV * 1024;
    static constexpr int X_HI = 2 * SPH, X_LO = X_HI + F::S32;
    static constexpr int Z_HI = X_LO + F::S32, Z_LO = Z_HI + F::ZOP;
    static constexpr int SB = Z_LO + F::ZOP;
};

template <int DV, int C, bool PREC, bool GATE>
constexpr int lds_fwd32() {
    using F = Cfg32<DV, C, GATE>;
    return PREC ? 2 * F::IO::BUF + Prec32<DV, C>::SB + F::NW * F::OTILE + F::NW * F::KROW
                : F::LDS_FWD;
}

template <int W, int PASS, int DV, int C>
__device__ __forceinline__ void publish_pass(char* sb, const State32<DV, C>& st, const Lane& L) {
    using F = Cfg32<DV, C>;
    using P = Prec32<DV, C>;
    if constexpr ((W < F::NW / 2) == (PASS == 0)) {
#pragma unroll
        for (int j = 0; j < F::TPW / 2; ++j)
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt) {
                const f32x4_t& x = st.s[2 * j][nt];
                const f32x4_t& y = st.s[2 * j + 1][nt];
                const int pl = F::TPW / 2 * W + j - 8 * PASS;
                const u32x4_t hi = {pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(y[0], y[1]), pk2(y[2], y[3])};
                const u32x2_t lx = lo_of(x, hi[0], hi[1]), ly = lo_of(y, hi[2], hi[3]);
                char* dst = sb + ((pl * F::NTV + nt) * 64 + L.lane) * 16;
                *reinterpret_cast<u32x4_t*>(dst) = hi;
                *reinterpret_cast<u32x4_t*>(dst + P::SPH) = u32x4_t{lx[0], lx[1], ly[0], ly[1]};
            }
    }
    if constexpr (PASS == 0) {
        if constexpr (has_x<DV, C, W>()) {
            const u32x2_t hi = {pk2(st.x[0], st.x[1]), pk2(st.x[2], st.x[3])};
            const int off = (xnt<DV, C, W>() * 64 + L.lane) * 8;
            *reinterpret_cast<u32x2_t*>(sb + P::X_HI + off) = hi;
            *reinterpret_cast<u32x2_t*>(sb + P::X_LO + off) = lo_of(st.x, hi[0], hi[1]);
        }
        if constexpr (W < 4) {
            constexpr int half = (W == 1 || W == 3) ? 1 : 0, part = W >= 2 ? 1 : 0;
            const u32x2_t hi = {pk2(st.z[0], st.z[1]), pk2(st.z[2], st.z[3])};
            const int off = (half * 64 + L.lane) * 16 + part * 8;
            *reinterpret_cast<u32x2_t*>(sb + P::Z_HI + off) = hi;
            *reinterpret_cast<u32x2_t*>(sb + P::Z_LO + off) = lo_of(st.z, hi[0], hi[1]);
        }
    }
}

// The inter-chunk numerator over the pairs of one pass as hi*hi + lo*hi + hi*lo
// (the lifted query is exact as hi + lo); pass 0 also takes tile 32 and returns
// this lane's part of q^T Z q (summed over the lane groups by the caller).
template <int PASS, int DV, int C>
__device__ __forceinline__ float inter_pass(const char* sb, const QueryRow& Q,
                                            f32x4_t (&num)[Cfg32<DV, C>::NTV + 1], const Lane& L) {
    using F = Cfg32<DV, C>;
    using P = Prec32<DV, C>;
    static_for<0, 8>([&](auto pc) {
        constexpr int pl = decltype(pc)::value;
        float f[8];
        query_pair_values<2 * (pl + 8 * PASS)>(Q, L, f);
        u32x4_t fh, fl;
        split8(f, fh, fl);
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) {
            const char* a = sb + ((pl * F::NTV + nt) * 64 + L.lane) * 16;
            const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(a);
            const u32x4_t al = *reinterpret_cast<const u32x4_t*>(a + P::SPH);
            num[nt] = mma32(ah, fh, num[nt]);
            num[nt] = mma32(al, fh, num[nt]);
            num[nt] = mma32(ah, fl, num[nt]);
        }
    });
    float d = 0.0f;
    if constexpr (PASS == 0) {
        const bool lo = L.g < 2;
        float f[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = query_entry<32>(Q, r, lo);
        u32x2_t fh, fl;
        split4(f, fh, fl);
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) {
            const int off = (nt * 64 + L.lane) * 8;
            const u32x2_t ah = *reinterpret_cast<const u32x2_t*>(sb + P::X_HI + off);
            const u32x2_t al = *reinterpret_cast<const u32x2_t*>(sb + P::X_LO + off);
            num[nt] = mma16_acc32(ah, fh, num[nt]);
            num[nt] = mma16_acc32(al, fh, num[nt]);
            num[nt] = mma16_acc32(ah, fl, num[nt]);
        }
        // Z q with Z as hi + lo (q is exact in bf16)
        const u32x4_t zlh = *reinterpret_cast<const u32x4_t*>(sb + P::Z_HI + L.lane * 16);
        const u32x4_t zuh = *reinterpret_cast<const u32x4_t*>(sb + P::Z_HI + (64 + L.lane) * 16);
        const u32x4_t zll = *reinterpret_cast<const u32x4_t*>(sb + P::Z_LO + L.lane * 16);
        const u32x4_t zul = *reinterpret_cast<const u32x4_t*>(sb + P::Z_LO + (64 + L.lane) * 16);
        const f32x4_t zl = mma32(zll, Q.zf, mma32(zlh, Q.zf, zero4()));
        const f32x4_t zu = mma32(zul, Q.zf, mma32(zuh, Q.zf, zero4()));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            d = __builtin_fmaf(Q.a[r], zl[r], d);
            d = __builtin_fmaf(Q.b[r], zu[r], d);
        }
    }
    return d;
}

// ---- per-wavefront bodies ----------------------------------------------------------

template <int W, int DV, int C, bool DECAY, bool PREC>
__device__ __forceinline__ void seg_state_body32(const bf16_t* k, const bf16_t* v, const float* gdec,
                                                 float* rec, float* segdec, char* lds, int T,
                                                 int NC, int G, int NSEG, const Lane& L) {
    using F = Cfg32<DV, C, DECAY>;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    LoadPipeline<DK, DV, C, F::NW, 4, DECAY> P{lds, seg * G, min(NC, seg * G + G), T, bh * T, gdec};
    float* krow = reinterpret_cast<float*>(lds + 4 * F::IO::BUF + W * F::KROW);
    float lsum = 0.0f;                             // log2 of the segment's decay
    State32<DV, C> st;
#pragma unroll
    for (int i = 0; i < F::TPW; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) st.s[i][nt] = zero4();
    st.x = zero4();
    st.z = zero4();

    P.prologue(k, v, L);
    for (int c = P.c0; c < P.c1; ++c) {
        P.acquire(k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::IO::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::IO::QB);
        KeyDecay kd{};
        if constexpr (DECAY) {
            kd = chunk_key_decays<C>(buf + 2 * F::IO::QB + F::IO::VB, krow, L);
            decay_state32<W, DV, C>(st, kd.last);
            lsum += kd.last;
        }
#pragma unroll
        for (int m = 0; m < F::KS; ++m) state_step<W, DV, C, DECAY, PREC>(st, bk, bv, m, L, kd);
        compiler_fence();
    }
    record_store32<W, DV, C>(rec + (bh * NSEG + seg) * (size_t)F::REC, st, L);
    if (DECAY && W == 0 && L.lane == 0) segdec[bh * NSEG + seg] = exp2_neg(lsum);
}

template <int W, int DV, int C, bool CAUSAL, bool DECAY, bool PREC>
__device__ __forceinline__ void fwd_body32(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                           const float* gdec, const float* prefix,
                                           float* final_rec, bf16_t* o, char* lds, int T, int NC,
                                           int G, int NSEG, const Lane& L) {
    using F = Cfg32<DV, C, DECAY>;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    // LDS: published state operands | two chunk buffers | output tiles | key
    // decays. The state operands come first: the workgroup's LDS starts at
    // address 0, so every state operand read of the first 64 KB is the lane's
    // base plus an immediate offset, with no address register per read.
    constexpr int SBX = PREC ? Prec32<DV, C>::SB : F::SB;   // published state operands
    char* sb = lds;
    Pipeline<DK, DV, C, F::NW, F::NW, DECAY> P{lds + SBX, seg * G, min(NC, seg * G + G), T, bh * T,
                                               true, gdec};
    char* otile = lds + SBX + 2 * F::IO::BUF + W * F::OTILE;
    float* krow = reinterpret_cast<float*>(lds + SBX + 2 * F::IO::BUF + F::NW * F::OTILE + W * F::KROW);

    State32<DV, C> st;
    record_load32<W, DV, C>(prefix + (CAUSAL ? bh * NSEG + seg : bh) * (size_t)F::REC, st, L);

    P.stage(q, k, v, P.c0, L);
    for (int c = P.c0; c < P.c1; ++c) {
        const int n = min(C, T - c * C);
        P.acquire(q, k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bq = reinterpret_cast<const bf16_t*>(buf);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::IO::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::IO::QB);
        KeyDecay kd{};
        if constexpr (DECAY) kd = chunk_key_decays<C>(buf + 2 * F::IO::QB + F::IO::VB, krow, L);

        // the state before this chunk, as bf16 operands for every wavefront (the
        // acquire barrier guarantees the previous chunk's readers are done);
        // split operands are published in two passes inside the tile loop
        if (!PREC && (CAUSAL || c == P.c0)) {
            publish_state<W, DV, C>(sb, st, L);
            lds_barrier();
        }

        // ---- per own query tile: inter-chunk term phi(Q).P and q^T Z q over the
        // published state, intra-chunk term, normalise, store. One tile at a time
        // keeps one query row and one set of accumulators live (the state
        // operands are read from LDS once per tile).
        bf16_t* oc = o + (bh * T + (size_t)c * C) * DV;
#pragma unroll
        for (int u = 0; u < F::TW; ++u) {
            const int tt = own_query_tile<W, F::TT, F::NW>(u);
            f32x4_t num[F::NTV + 1];
#pragma unroll
            for (int nt = 0; nt <= F::NTV; ++nt) num[nt] = zero4();
            float di;
            if constexpr (PREC) {
                static_assert(F::TW == 1, "one query tile per wavefront");
                QueryRow Q;
                load_query32(bq, tt, L, Q);
                publish_pass<W, 0, DV, C>(sb, st, L);
                lds_barrier();
                float d = inter_pass<0, DV, C>(sb, Q, num, L);
                lds_barrier();                            // pass 0 read by everyone
                publish_pass<W, 1, DV, C>(sb, st, L);
                lds_barrier();
                inter_pass<1, DV, C>(sb, Q, num, L);
                d += __shfl_xor(d, 16, 64);
                d += __shfl_xor(d, 32, 64);
                di = d;
            } else {
                QueryRow Q;
                load_query32(bq, tt, L, Q);
                static_for<0, 16>([&](auto pc) {
                    constexpr int p = decltype(pc)::value;
                    const u32x4_t fq = lift_query_pair<2 * p>(Q, L);
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) {
                        const u32x4_t a =
                            *reinterpret_cast<const u32x4_t*>(sb + ((p * F::NTV + nt) * 64 + L.lane) * 16);
                        num[nt] = mma32(a, fq, num[nt]);
                    }
                });
                {
                    const u32x2_t fq = lift_query_mixed(Q, L);
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) {
                        const u32x2_t a =
                            *reinterpret_cast<const u32x2_t*>(sb + F::SPAIR + (nt * 64 + L.lane) * 8);
                        num[nt] = mma16_acc32(a, fq, num[nt]);
                    }
                }
                const char* zb = sb + F::SPAIR + F::S32;
                const u32x4_t zal = *reinterpret_cast<const u32x4_t*>(zb + L.lane * 16);
                const u32x4_t zau = *reinterpret_cast<const u32x4_t*>(zb + (64 + L.lane) * 16);
                const f32x4_t zl = mma32(zal, Q.zf, zero4());
                const f32x4_t zu = mma32(zau, Q.zf, zero4());
                float d = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    d = __builtin_fmaf(Q.a[r], zl[r], d);
                    d = __builtin_fmaf(Q.b[r], zu[r], d);
                }
                d += __shfl_xor(d, 16, 64);
                d += __shfl_xor(d, 32, 64);
                di = d;
            }
            float bt = 0.0f;                              // b of this lane's query
            if constexpr (DECAY) {                        // the prefix state decays to query t
                bt = krow[16 * tt + L.c16];
                const float e = exp2_neg(bt);
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) num[nt] *= e;
                di *= e;
            }
            // ---- intra-chunk term: A = (Q K^T)^2 masked to j <= t, num += A [V | 1]
            if (CAUSAL) {
                const int t = 16 * tt + L.c16;
                const u32x4_t qf = lds_row<2 * DK, u32x4_t>(bq, t, 16 * L.g);
                const u32x4_t ones = ones_op(L);
                for (int m = 0; m <= tt / 2; ++m) {
                    const bool diag = 32 * m + 31 > 16 * tt;
                    float w[8];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x4_t kf =
                            lds_row<2 * DK, u32x4_t>(bk, 32 * m + 16 * h + L.c16, 16 * L.g);
                        // rows j = 32m + 16h + 4g + r, column t
                        const f32x4_t sc = mma32(kf, qf, zero4());
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = 32 * m + 16 * h + 4 * L.g + r;
                            float x = sc[r] * sc[r];
                            if constexpr (DECAY) x *= exp2_neg(bt - kd.b(2 * m + h, r));
                            w[4 * h + r] = (!diag || j <= t) ? x : 0.0f;
                        }
                    }
                    const u32x4_t at = pack8(w);
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt)
                        num[nt] = mma32(v_fragment_tr<DV>(bv, m, nt, L), at, num[nt]);
                    num[F::NTV] = mma32(ones, at, num[F::NTV]);
                }
            }
            // ---- normalise and store: o = num / den
            {
                // intra-chunk denominator: row 0 of the ones tile (lane group 0)
                const float den = __shfl(num[F::NTV][0], L.c16, 64) + di;
                const float y = inv_den(den);                  // y = 0 gives o = 0
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) {
                    float ov[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ov[r] = num[nt][r] * y;
                    }
                    *reinterpret_cast<u32x2_t*>(otile + L.c16 * F::OROW + 2 * (16 * nt + 4 * L.g)) =
                        u32x2_t{pk2(ov[0], ov[1]), pk2(ov[2], ov[3])};
                }
                compiler_fence();                         // staged rows written before read back
#pragma unroll
                for (int i = 0; i < (F::OU + 63) / 64; ++i) {
                    const int unit = L.lane + 64 * i;
                    const int row = unit / (F::OU / 16), col = unit % (F::OU / 16);
                    if (unit < F::OU) {
                        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(otile + row * F::OROW + 16 * col);
                        if (16 * tt + row < n)
                            store16(oc, (uint32_t)(((16 * tt + row) * DV + 8 * col) * 2), val);
                    }
                }
                compiler_fence();                         // read back before the next tile's rows
            }
        }

        // ---- running state: S += phi(K_c)^T V_c, Z += K_c^T K_c (not needed
        // after the segment's last chunk unless the final state is asked for)
        if (CAUSAL && (c + 1 < P.c1 || final_rec)) {
            if constexpr (DECAY) decay_state32<W, DV, C>(st, kd.last);
#pragma unroll
            for (int m = 0; m < F::KS; ++m) state_step<W, DV, C, DECAY, PREC>(st, bk, bv, m, L, kd);
        }
        compiler_fence();
    }
    // running state after the segment's last chunk (one segment per head: the
    // final state), when asked for
    if (CAUSAL && final_rec) record_store32<W, DV, C>(final_rec + bh * (size_t)F::REC, st, L);
}

// Body dispatch by wavefront index (compile-time roles).
template <int DV, int C, typename F>
__device__ __forceinline__ void by_wave(int w, F&& f) {
    static_for<0, Cfg32<DV, C>::NW>([&](auto wc) {
        if (w == decltype(wc)::value) f(wc);
    });
}

// ---- kernels -------------------------------------------------------------------

template <int DV, int C, bool DECAY, bool PREC>
__global__ __launch_bounds__(kThreads32<C>, kWavesPerSimd32<C>)
void kata_seg_state32(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                      const float* __restrict__ gdec, float* __restrict__ rec,
                      float* __restrict__ segdec, int T, int NC, int G, int NSEG) {
    using F = Cfg32<DV, C, DECAY>;
    __shared__ __attribute__((aligned(16))) char lds[F::LDS_SEG];
    const Lane L;
    by_wave<DV, C>(L.w, [&](auto wc) {
        seg_state_body32<decltype(wc)::value, DV, C, DECAY, PREC>(k, v, gdec, rec, segdec, lds, T, NC,
                                                            G, NSEG, as_wave<decltype(wc)::value>(L));
    });
}

template <int DV, int C, bool CAUSAL, bool DECAY, bool PREC>
__global__ __launch_bounds__(kThreads32<C>, kWavesPerSimd32<C>)
void kata_fwd32(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, const float* __restrict__ gdec,
                const float* __restrict__ prefix, float* __restrict__ final_rec,
                bf16_t* __restrict__ o, int T, int NC, int G, int NSEG) {
    constexpr int kLds = lds_fwd32<DV, C, PREC, DECAY>();
    static_assert(kLds <= 160 * 1024, "fits the LDS of a compute unit");
    __shared__ __attribute__((aligned(16))) char lds[kLds];
    const Lane L;
    by_wave<DV, C>(L.w, [&](auto wc) {
        fwd_body32<decltype(wc)::value, DV, C, CAUSAL, DECAY, PREC>(q, k, v, gdec, prefix, final_rec, o,
                                                              lds, T, NC, G, NSEG,
                                                              as_wave<decltype(wc)::value>(L));
    });
}

// Launch arguments shared by every shape: gdec (log-decays, NULL = no gate;
// causal only), segdec (per-segment decays, state kernel), rec (segment
// records for the state kernel, the final-state records for the output
// kernel).
struct Args32 {
    const void *q, *k, *v;
    const float* gdec;
    float* rec;
    float* segdec;
    const float* prefix;
    void* o;
    int causal, G, NSEG;
    bool state_only;
    bool prec;             // split operands (the gated kernels always take them)
};

template <int DV, int C>
hipError_t launch_dv_c32(const Shape& s, const Args32& a, hipStream_t st) {
    dim3 grid(a.NSEG, s.B * s.H);
    constexpr int threads = kThreads32<C>;
    const bf16_t *q = (const bf16_t*)a.q, *k = (const bf16_t*)a.k, *v = (const bf16_t*)a.v;
    bf16_t* o = (bf16_t*)a.o;
    if (a.gdec && !a.causal) return hipErrorInvalidValue;
    if (a.state_only) {
        if (a.gdec)
            kata_seg_state32<DV, C, true, true><<<grid, threads, 0, st>>>(k, v, a.gdec, a.rec, a.segdec,
                                                                           s.T, s.NC, a.G, a.NSEG);
        else if (a.prec)
            kata_seg_state32<DV, C, false, true><<<grid, threads, 0, st>>>(k, v, nullptr, a.rec, nullptr,
                                                                            s.T, s.NC, a.G, a.NSEG);
        else
            kata_seg_state32<DV, C, false, false><<<grid, threads, 0, st>>>(k, v, nullptr, a.rec, nullptr,
                                                                             s.T, s.NC, a.G, a.NSEG);
    } else if (a.gdec) {
        kata_fwd32<DV, C, true, true, true><<<grid, threads, 0, st>>>(q, k, v, a.gdec, a.prefix, a.rec, o,
                                                                       s.T, s.NC, a.G, a.NSEG);
    } else if (a.causal) {
        if (a.prec)
            kata_fwd32<DV, C, true, false, true><<<grid, threads, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                            a.rec, o, s.T, s.NC, a.G, a.NSEG);
        else
            kata_fwd32<DV, C, true, false, false><<<grid, threads, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                             a.rec, o, s.T, s.NC, a.G, a.NSEG);
    } else {
        if (a.prec)
            kata_fwd32<DV, C, false, false, true><<<grid, threads, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                             a.rec, o, s.T, s.NC, a.G, a.NSEG);
        else
            kata_fwd32<DV, C, false, false, false><<<grid, threads, 0, st>>>(q, k, v, nullptr, a.prefix,
                                                                              a.rec, o, s.T, s.NC, a.G, a.NSEG);
    }
    return hipGetLastError();
}

template <int C>
hipError_t launch_c32(const Shape& s, const Args32& a, hipStream_t st) {
    switch (s.dv) {
        case 16: return launch_dv_c32<16, C>(s, a, st);
        case 32: return launch_dv_c32<32, C>(s, a, st);
        case 64: return launch_dv_c32<64, C>(s, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch32(const Shape& s, const Args32& a, hipStream_t st) {
    switch (s.C) {
        case 64: return launch_c32<64>(s, a, st);
        case 128: return launch_c32<128>(s, a, st);
    }
    return hipErrorInvalidValue;
}

// ---- per-chunk exclusive prefixes (kata_scan_states) -------------------------------
// As at d_k = 16: one workgroup per segment walks its chunks from the segment's
// scanned prefix, writes each chunk's exclusive prefix to the packed
// S_prefix[c], z_prefix[c], then adds the chunk with split key operands.
// Wavefront w writes the tiles, the tile-32 value tile and the Gram tile it
// owns (its lower-triangle entries skipped).

template <int W, int DV, int C>
__device__ __forceinline__ void store_packed32(const State32<DV, C>& st, float* Sp, float* zp,
                                               const Lane& L) {
    using F = Cfg32<DV, C>;
    auto put = [&](int tile, int nt, const f32x4_t& x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int col;
            float scale;
            bool lower;
            const int p = rec32_to_packed(((tile * F::NTV + nt) * 64 + L.lane) * 4 + r, F::NTV,
                                          &col, &scale, &lower);
            Sp[p * DV + col] = x[r] * scale;
        }
    };
#pragma unroll
    for (int i = 0; i < F::TPW; ++i)
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) put(F::TPW * W + i, nt, st.s[i][nt]);
    if constexpr (has_x<DV, C, W>()) put(32, xnt<DV, C, W>(), st.x);
    if constexpr (W < 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int col;
            float scale;
            bool lower;
            const int p = rec32_to_packed(NFT * F::NTV * 256 + (W * 64 + L.lane) * 4 + r, F::NTV,
                                          &col, &scale, &lower);
            if (!lower) zp[p] = st.z[r] * scale;
        }
    }
}

template <int W, int DV, int C>
__device__ __forceinline__ void prefix_body32(const bf16_t* k, const bf16_t* v, const float* prefix,
                                              float* Sp, float* zp, char* lds, int T, int NC,
                                              int G, int NSEG, const Lane& L) {
    using F = Cfg32<DV, C>;
    constexpr int D = DK * (DK + 1) / 2;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int c0 = seg * G, c1 = min(NC, seg * G + G);
    LoadPipeline<DK, DV, C, F::NW, 4, false> P{lds, c0, c1 - 1, T, bh * T, nullptr};
    State32<DV, C> st;
    record_load32<W, DV, C>(prefix + (bh * NSEG + seg) * (size_t)F::REC, st, L);
    P.prologue(k, v, L);
    for (int c = c0; c < c1 - 1; ++c) {
        store_packed32<W, DV, C>(st, Sp + (bh * NC + c) * (size_t)(D * DV), zp + (bh * NC + c) * (size_t)D, L);
        P.acquire(k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::IO::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::IO::QB);
#pragma unroll
        for (int m = 0; m < F::KS; ++m) state_step<W, DV, C, false, true>(st, bk, bv, m, L);
        compiler_fence();
    }
    store_packed32<W, DV, C>(st, Sp + (bh * NC + c1 - 1) * (size_t)(D * DV),
                             zp + (bh * NC + c1 - 1) * (size_t)D, L);
}

template <int DV, int C>
__global__ __launch_bounds__(kThreads32<C>, kWavesPerSimd32<C>)
void kata_prefix32(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                   const float* __restrict__ prefix, float* __restrict__ Sp,
                   float* __restrict__ zp, int T, int NC, int G, int NSEG) {
    using F = Cfg32<DV, C>;
    __shared__ __attribute__((aligned(16))) char lds[F::LDS_SEG];
    const Lane L;
    by_wave<DV, C>(L.w, [&](auto wc) {
        prefix_body32<decltype(wc)::value, DV, C>(k, v, prefix, Sp, zp, lds, T, NC, G, NSEG,
                                                  as_wave<decltype(wc)::value>(L));
    });
}

template <int C>
hipError_t launch_prefix32_c(const Shape& s, const void* k, const void* v, const float* prefix,
                             float* Sp, float* zp, int G, int NSEG, hipStream_t st) {
    dim3 grid(NSEG, s.B * s.H);
    constexpr int threads = kThreads32<C>;
    const bf16_t *kk = (const bf16_t*)k, *vv = (const bf16_t*)v;
    switch (s.dv) {
        case 16: kata_prefix32<16, C><<<grid, threads, 0, st>>>(kk, vv, prefix, Sp, zp, s.T, s.NC, G, NSEG); break;
        case 32: kata_prefix32<32, C><<<grid, threads, 0, st>>>(kk, vv, prefix, Sp, zp, s.T, s.NC, G, NSEG); break;
        case 64: kata_prefix32<64, C><<<grid, threads, 0, st>>>(kk, vv, prefix, Sp, zp, s.T, s.NC, G, NSEG); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

__global__ void record_from_packed32(float* __restrict__ rec, const float* __restrict__ S,
                                     const float* __restrict__ z, int NTV, int REC, int nrec) {
    const int D = DK * (DK + 1) / 2, DV = 16 * NTV;
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        int col;
        float scale;
        bool lower;
        const int p = rec32_to_packed((int)(x % REC), NTV, &col, &scale, &lower);
        rec[x] = (col >= 0 ? S[(b * D + p) * DV + col] : z[b * D + p]) / scale;
    }
}

__global__ void record_to_packed32_kernel(const float* __restrict__ rec, float* __restrict__ S,
                                          float* __restrict__ z, int NTV, int REC, int nrec) {
    const int D = DK * (DK + 1) / 2, DV = 16 * NTV;
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        int col;
        float scale;
        bool lower;
        const int p = rec32_to_packed((int)(x % REC), NTV, &col, &scale, &lower);
        if (lower) continue;
        const float val = rec[x] * scale;
        if (col >= 0) S[(b * D + p) * DV + col] = val;
        else z[b * D + p] = val;
    }
}

}  // namespace

bool mfma32_supported(const Shape& s) {
    return s.bf16 && s.dk == 32 && (s.C == 64 || s.C == 128) &&
           (s.dv == 16 || s.dv == 32 || s.dv == 64);
}

int mfma32_record_floats(int dv) { return NFT * (dv / 16) * 256 + NZ * 256; }

hipError_t launch_seg_state32(const Shape& s, const void* k, const void* v, float* rec, int G,
                              int NSEG, bool prec, hipStream_t st) {
    return dispatch32(s, Args32{nullptr, k, v, nullptr, rec, nullptr, nullptr, nullptr, 1, G, NSEG, true,
                                prec}, st);
}

hipError_t launch_fwd32(const Shape& s, const void* q, const void* k, const void* v,
                        const float* prefix, float* final_rec, void* o, int causal, int G,
                        int NSEG, bool prec, hipStream_t st) {
    return dispatch32(s, Args32{q, k, v, nullptr, final_rec, nullptr, prefix, o, causal, G, NSEG, false,
                                prec}, st);
}

hipError_t launch_seg_state32_decay(const Shape& s, const void* k, const void* v, const float* gdec,
                                    float* rec, float* segdec, int G, int NSEG, hipStream_t st) {
    return dispatch32(s, Args32{nullptr, k, v, gdec, rec, segdec, nullptr, nullptr, 1, G, NSEG, true, true},
                      st);
}

hipError_t launch_fwd32_decay(const Shape& s, const void* q, const void* k, const void* v,
                              const float* gdec, const float* prefix, float* final_rec, void* o,
                              int G, int NSEG, hipStream_t st) {
    return dispatch32(s, Args32{q, k, v, gdec, final_rec, nullptr, prefix, o, 1, G, NSEG, false, true}, st);
}

hipError_t launch_prefix32(const Shape& s, const void* k, const void* v, const float* prefix,
                           float* Sp, float* zp, int G, int NSEG, hipStream_t st) {
    switch (s.C) {
        case 64: return launch_prefix32_c<64>(s, k, v, prefix, Sp, zp, G, NSEG, st);
        case 128: return launch_prefix32_c<128>(s, k, v, prefix, Sp, zp, G, NSEG, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_record_from_packed32(float* rec, const float* S, const float* z, int dv,
                                       int nrec, hipStream_t st) {
    const int REC = mfma32_record_floats(dv);
    const size_t n = (size_t)REC * nrec;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    record_from_packed32<<<blocks, 256, 0, st>>>(rec, S, z, dv / 16, REC, nrec);
    return hipGetLastError();
}

hipError_t launch_record_to_packed32(const float* rec, float* S, float* z, int dv, int nrec,
                                     hipStream_t st) {
    const int REC = mfma32_record_floats(dv);
    const size_t n = (size_t)REC * nrec;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    record_to_packed32_kernel<<<blocks, 256, 0, st>>>(rec, S, z, dv / 16, REC, nrec);
    return hipGetLastError();
}

}  // namespace kata
