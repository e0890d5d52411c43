// Factored PSD features, KATA-Mg and KATA-Sigma-g: chunked forward and state
// build on gfx950 matrix cores.
//
// The KATA explainers (gist.science, technical summary 2.3, "Variants") name
// KATA-Mg (multiple PSD factors) and KATA-Sigma-g (summed PSD factors), which
// trade state size against packing efficiency, without a construction. Reading
// built here: a query or key x of width d_k is cut into G contiguous factors
// x_a = x[aP, (a+1)P), P = d_k / G, each lifted to the rank-one PSD matrix
// x_a x_a^T of technical summary 2.2.
//   multi  (Mg):      the factors stay apart - the block-diagonal feature
//                     diag(x_1 x_1^T, ..., x_G x_G^T), D = G P(P+1)/2 entries,
//                     weight sum_a (q_a . k_a)^2;
//   summed (Sigma-g): the factors are summed into one P x P matrix
//                     sum_a x_a x_a^T, D = P(P+1)/2 entries,
//                     weight sum_{a,b} (q_a . k_b)^2.
// Feature f is the packed entry of the boundary's layout (row-major upper
// triangle of a factor, sqrt(2) off the diagonal; multi: factor a at
// [a P(P+1)/2, (a+1) P(P+1)/2)), so records map to the packed state row for
// row.
//
// The chunked-state form and its pieces are those of the plain lift: segment
// states of G_seg chunks, an associative scan over segment records, and an
// output kernel that walks its segment from the scanned prefix with the masked
// intra-chunk term.
//
// Precision. The intra-chunk weights come from the factors' inner products,
// formed on the matrix cores from the bf16 inputs (exact products, fp32 sums)
// and squared in fp32: a factor pair (a, b) is one product of the query
// fragment masked to factor a with the key fragment read rotated by (b - a) P
// elements. The lifted features and the state enter the matrix cores as split
// bf16 operands (hi + lo, about 16 significant bits), so the inter-chunk term
// keeps its accuracy however few keys the prefix holds.
//
// Work split: four wavefronts. Feature tile at (16 features) belongs to
// wavefront at % 4, which holds its state units (value tiles and the z tile)
// in registers, lifts its keys and updates them; before a chunk's outputs the
// owners publish the state as split bf16 operands to LDS, and wavefront w
// evaluates query tile w of the chunk (inter-chunk term from the published
// state, intra-chunk term, normalisation, store).
#include <algorithm>
#include <type_traits>
#include <utility>

#include "kata_chunk.h"
#include "kata_internal.h"
#include "kata_records.h"

namespace kata {

namespace {

constexpr int NWF = 4;                 // wavefronts per workgroup

template <int DK_, int G_, bool SUMMED_>
struct Fact {
    static constexpr int DK = DK_, G = G_;
    static constexpr bool SUMMED = SUMMED_;
    static constexpr int P = DK / G;               // factor width
    static constexpr int NF = P * (P + 1) / 2;     // packed entries of one factor's lift
    static constexpr int D = SUMMED ? NF : G * NF; // feature dimension
    static constexpr int NAT = (D + 15) / 16;      // feature tiles
    static constexpr int NPAIR = (NAT + 1) / 2;    // K = 32 operand pairs of tiles
    static constexpr int NOWN = (NAT + NWF - 1) / NWF;   // tiles per wavefront (at most)
    static constexpr int EPL = DK / 4;             // row elements per lane group (scores)
    static_assert(DK % G == 0 && P >= EPL, "a lane group's elements lie in one factor");
};

// Factor (multi: its index; summed: 0) and element pair (i <= j, within the
// factor) of feature f < D in the packed order (compile-time for the lifts).
template <class F>
__host__ __device__ constexpr void feature_pair(int f, int* a, int* i, int* j) {
    *a = F::SUMMED ? 0 : f / F::NF;
    int r = f % F::NF, row = 0;
    while (r >= F::P - row) {                      // row `row` holds P - row entries
        r -= F::P - row;
        ++row;
    }
    *i = row;
    *j = row + r;
}

// Lifted rows of the chunk in LDS: per feature tile, [C][16] bf16 rows (32
// bytes, swizzled as staged rows) of the hi and the lo parts, keys then
// queries. Key tiles are read as transposed A fragments of the state update,
// query tiles as B fragments of the inter-chunk term.
template <int C, int NP>
struct Lifted {
    static constexpr int TILE = C * 32;            // bytes of one [C][16] bf16 tile
    // part: 0 key hi, 1 key lo, 2 query hi, 3 query lo (NP = 2: keys only)
    __device__ static const bf16_t* tile(const char* base, int at, int part) {
        return reinterpret_cast<const bf16_t*>(base + (NP * at + part) * TILE);
    }
    __device__ static char* tile_w(char* base, int at, int part) { return base + (NP * at + part) * TILE; }
};

// The staged row r (DK bf16, swizzled) as fp32.
template <int DK>
__device__ __forceinline__ void load_row(const bf16_t* rows, int r, float (&x)[DK]) {
#pragma unroll
    for (int u = 0; u < DK / 8; ++u) {
        const u32x4_t w = lds_row<2 * DK, u32x4_t>(rows, r, 16 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[8 * u + 2 * e] = lo_bf16(w[e]);
            x[8 * u + 2 * e + 1] = hi_bf16(w[e]);
        }
    }
}

// Feature f of a row x (fp32; products of bf16 values are exact, a summed
// feature adds the G factors' products), f compile-time.
template <class F, int f>
__device__ __forceinline__ float lift_value(const float (&x)[F::DK]) {
    if constexpr (f >= F::D) {
        return 0.0f;
    } else {
        constexpr int a = [] { int a_ = 0, i_ = 0, j_ = 0; feature_pair<F>(f, &a_, &i_, &j_); return a_; }();
        constexpr int i = [] { int a_ = 0, i_ = 0, j_ = 0; feature_pair<F>(f, &a_, &i_, &j_); return i_; }();
        constexpr int j = [] { int a_ = 0, i_ = 0, j_ = 0; feature_pair<F>(f, &a_, &i_, &j_); return j_; }();
        float acc;
        if constexpr (F::SUMMED) {
            acc = 0.0f;
#pragma unroll
            for (int b = 0; b < F::G; ++b) acc += x[b * F::P + i] * x[b * F::P + j];
        } else {
            acc = x[a * F::P + i] * x[a * F::P + j];
        }
        return i != j ? acc * kSqrt2 : acc;
    }
}

// Tile AT (features 16 AT .. 16 AT + 15) of row r: split into hi and lo and
// written as two 32-byte rows.
template <class F, int AT, int... c>
__device__ __forceinline__ void lift16(const float (&x)[F::DK], float (&f)[16],
                                       std::integer_sequence<int, c...>) {
    ((f[c] = lift_value<F, 16 * AT + c>(x)), ...);
}

template <class F, int C, int NP, int AT>
__device__ __forceinline__ void lift_tile(const float (&x)[F::DK], char* lifted, int r, int part0) {
    float f[16];
    lift16<F, AT>(x, f, std::make_integer_sequence<int, 16>{});
    u32x4_t hi[2], lo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float g8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) g8[e] = f[8 * h + e];
        split8(g8, hi[h], lo[h]);
    }
    char* th = Lifted<C, NP>::tile_w(lifted, AT, part0);
    char* tl = Lifted<C, NP>::tile_w(lifted, AT, part0 + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<u32x4_t*>(th + Swz<32>::off(r, 16 * h)) = hi[h];
        *reinterpret_cast<u32x4_t*>(tl + Swz<32>::off(r, 16 * h)) = lo[h];
    }
}

// Tiles R, R + 4, ... of row r.
template <class F, int C, int NP, int R>
__device__ __forceinline__ void lift_tiles(const float (&x)[F::DK], char* lifted, int r, int part0) {
    if constexpr (R < F::NAT) {
        lift_tile<F, C, NP, R>(x, lifted, r, part0);
        lift_tiles<F, C, NP, R + 4>(x, lifted, r, part0);
    }
}

// The lifted key (WITH_K) and query (WITH_Q) tiles of the staged chunk:
// thread t takes row t / 4 and the tiles congruent to t % 4 modulo 4.
template <class F, int C, int NP, bool WITH_K, bool WITH_Q>
__device__ __forceinline__ void lift_chunk(const bf16_t* bq, const bf16_t* bk, char* lifted, int tid) {
    static_assert(C * 4 == 64 * NWF, "four threads per row");
    const int r = tid >> 2, q4 = tid & 3;
    float x[F::DK];
    if constexpr (WITH_K) {
        load_row<F::DK>(bk, r, x);
        switch (q4) {
            case 0: lift_tiles<F, C, NP, 0>(x, lifted, r, 0); break;
            case 1: lift_tiles<F, C, NP, 1>(x, lifted, r, 0); break;
            case 2: lift_tiles<F, C, NP, 2>(x, lifted, r, 0); break;
            default: lift_tiles<F, C, NP, 3>(x, lifted, r, 0); break;
        }
    }
    if constexpr (WITH_Q) {
        load_row<F::DK>(bq, r, x);
        switch (q4) {
            case 0: lift_tiles<F, C, NP, 0>(x, lifted, r, 2); break;
            case 1: lift_tiles<F, C, NP, 1>(x, lifted, r, 2); break;
            case 2: lift_tiles<F, C, NP, 2>(x, lifted, r, 2); break;
            default: lift_tiles<F, C, NP, 3>(x, lifted, r, 2); break;
        }
    }
}

// The B operand slots of tile pair P2 for lane group G4 of a query row x:
// slot s is feature 16 (2 P2 + s / 4) + 4 G4 + s % 4 (compile-time pairs).
template <class F, int P2, int G4, int... s>
__device__ __forceinline__ void query_slots(const float (&x)[F::DK], float (&f)[8],
                                            std::integer_sequence<int, s...>) {
    ((f[s] = lift_value<F, 16 * (2 * P2 + s / 4) + 4 * G4 + s % 4>(x)), ...);
}
template <class F, int P2>
__device__ __forceinline__ void query_feats(const float (&x)[F::DK], int g, float (&f)[8]) {
    switch (g) {
        case 0: query_slots<F, P2, 0>(x, f, std::make_integer_sequence<int, 8>{}); break;
        case 1: query_slots<F, P2, 1>(x, f, std::make_integer_sequence<int, 8>{}); break;
        case 2: query_slots<F, P2, 2>(x, f, std::make_integer_sequence<int, 8>{}); break;
        default: query_slots<F, P2, 3>(x, f, std::make_integer_sequence<int, 8>{}); break;
    }
}

// Running state of one wavefront: units (tile W + 4 o, u), u = DV/16 the z
// tile (against the ones operand: column 0 holds z). Element r of lane (c16, g)
// of unit (at, u) is S[16 at + 4 g + r][16 u + c16].
template <class F, int DV>
struct FState {
    f32x4_t s[F::NOWN][DV / 16 + 1];
};

template <int W, class F>
__host__ __device__ constexpr bool owned(int o) {
    return W + NWF * o < F::NAT;
}

template <int W, class F, int DV>
__device__ __forceinline__ void state_zero(FState<F, DV>& st) {
#pragma unroll
    for (int o = 0; o < F::NOWN; ++o)
#pragma unroll
        for (int u = 0; u <= DV / 16; ++u) st.s[o][u] = zero4();
}

// S += phi(K_c)^T [V_c | 1] for the wavefront's tiles: A = lifted keys (lane
// c16 = feature, slots = tokens 32m + 16(s/4) + 4g + s%4), read transposed from
// the lifted hi and lo tiles, against exact bf16 V^T fragments or the ones
// operand.
template <int W, class F, int DV, int C, int NP>
__device__ __forceinline__ void state_update(FState<F, DV>& st, const char* lifted,
                                             const bf16_t* bv, const Lane& L) {
    constexpr int NTV = DV / 16, NU = NTV + 1;
    const u32x4_t ones = ones_op(L);
#pragma unroll
    for (int m = 0; m < C / 32; ++m) {
        u32x4_t b[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) b[u] = u < NTV ? v_fragment_tr<DV>(bv, m, u, L) : ones;
#pragma unroll
        for (int o = 0; o < F::NOWN; ++o) {
            if (!owned<W, F>(o)) continue;
            const int at = W + NWF * o;
            const u32x4_t hi = v_fragment_tr<16>(Lifted<C, NP>::tile(lifted, at, 0), m, 0, L);
            const u32x4_t lo = v_fragment_tr<16>(Lifted<C, NP>::tile(lifted, at, 1), m, 0, L);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                st.s[o][u] = mma32(hi, b[u], st.s[o][u]);
                st.s[o][u] = mma32(lo, b[u], st.s[o][u]);
            }
        }
    }
}

// Record of a state: unit (at, u) at (at * NU + u) * 256 floats, lane-major.
template <int W, class F, int DV>
__device__ __forceinline__ void record_store(float* rec, const FState<F, DV>& st, const Lane& L) {
    constexpr int NU = DV / 16 + 1;
    f32x4_t* r4 = reinterpret_cast<f32x4_t*>(rec);
#pragma unroll
    for (int o = 0; o < F::NOWN; ++o)
        if (owned<W, F>(o))
#pragma unroll
            for (int u = 0; u < NU; ++u) r4[((W + NWF * o) * NU + u) * 64 + L.lane] = st.s[o][u];
}

template <int W, class F, int DV>
__device__ __forceinline__ void record_load(const float* rec, FState<F, DV>& st, const Lane& L) {
    constexpr int NU = DV / 16 + 1;
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(rec);
#pragma unroll
    for (int o = 0; o < F::NOWN; ++o)
#pragma unroll
        for (int u = 0; u < NU; ++u)
            st.s[o][u] = owned<W, F>(o) ? r4[((W + NWF * o) * NU + u) * 64 + L.lane] : zero4();
}

// Published state: A operands of S^T (rows = value columns, K = features) for
// every tile pair p and unit u, 64 lanes x 16 bytes each; slots 0..3 are tile
// 2p (features 32p + 4g + s), slots 4..7 tile 2p + 1. The hi words, then the
// lo words.
template <class F, int DV>
struct Pub {
    static constexpr int NU = DV / 16 + 1;
    static constexpr int BYTES = F::NPAIR * NU * 1024;   // one of hi, lo
    __device__ static int off(int p, int u, int lane) { return (p * NU + u) * 1024 + lane * 16; }
};

template <int W, class F, int DV>
__device__ __forceinline__ void publish(const FState<F, DV>& st, char* pub, const Lane& L) {
    using PB = Pub<F, DV>;
#pragma unroll
    for (int o = 0; o < F::NOWN; ++o) {
        if (!owned<W, F>(o)) continue;
        const int at = W + NWF * o;
#pragma unroll
        for (int u = 0; u < PB::NU; ++u) {
            const f32x4_t& x = st.s[o][u];
            const uint32_t h0 = pk2(x[0], x[1]), h1 = pk2(x[2], x[3]);
            const int off = PB::off(at / 2, u, L.lane) + 8 * (at & 1);
            *reinterpret_cast<u32x2_t*>(pub + off) = u32x2_t{h0, h1};
            *reinterpret_cast<u32x2_t*>(pub + PB::BYTES + off) = lo_of(x, h0, h1);
        }
    }
}

// num[u] += S^T (published, split) . phi(q) (split) over tile pair P2.
template <class F, int DV, int P2>
__device__ __forceinline__ void inter_pair(const float (&x)[F::DK], const char* pub,
                                           f32x4_t (&num)[DV / 16 + 1], const Lane& L) {
    using PB = Pub<F, DV>;
    float f[8];
    query_feats<F, P2>(x, L.g, f);
    u32x4_t qh, ql;
    split8(f, qh, ql);
#pragma unroll
    for (int u = 0; u < PB::NU; ++u) {
        const int off = PB::off(P2, u, L.lane);
        const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(pub + off);
        const u32x4_t al = *reinterpret_cast<const u32x4_t*>(pub + PB::BYTES + off);
        num[u] = mma32(ah, qh, num[u]);
        num[u] = mma32(ah, ql, num[u]);
        num[u] = mma32(al, qh, num[u]);
    }
}
template <class F, int DV, int... P2>
__device__ __forceinline__ void inter_pairs(const float (&x)[F::DK], const char* pub,
                                            f32x4_t (&num)[DV / 16 + 1], const Lane& L,
                                            std::integer_sequence<int, P2...>) {
    (inter_pair<F, DV, P2>(x, pub, num, L), ...);
}

// Scores of 16 keys (staged rows krow .. +15: lane c16 = key) against this
// lane's query: D[key 4g + r][query c16] = the weight of that pair, sum over
// factor pairs of their squared inner products.
template <class F>
__device__ __forceinline__ f32x4_t weights16(const bf16_t* bk, int krow,
                                             const typename std::conditional<F::DK == 16, u32x2_t, u32x4_t>::type& qf,
                                             const Lane& L) {
    using Frag = typename std::conditional<F::DK == 16, u32x2_t, u32x4_t>::type;
    const int fac = L.g * F::EPL / F::P;           // factor of this lane group's elements
    f32x4_t w = zero4();
#pragma unroll
    for (int r = 0; r < (F::SUMMED ? F::G : 1); ++r) {
        // key elements (g EPL + r P) mod DK: factor a + r against the query's factor a
        const Frag kf = lds_row<2 * F::DK, Frag>(bk, krow, 2 * ((L.g * F::EPL + r * F::P) % F::DK));
#pragma unroll
        for (int a = 0; a < F::G; ++a) {
            Frag qa;
#pragma unroll
            for (int i = 0; i < (int)(sizeof(Frag) / 4); ++i) qa[i] = fac == a ? qf[i] : 0u;
            f32x4_t s;
            if constexpr (F::DK == 16) s = mma16(kf, qa, zero4());
            else s = mma32(kf, qa, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] += s[e] * s[e];
        }
    }
    return w;
}

// ---- segment states ----------------------------------------------------------

template <int W, class F, int DV, int C>
__device__ __forceinline__ void seg_state_body(const bf16_t* k, const bf16_t* v, float* rec,
                                               char* lds, int T, int NC, int Gs, int NSEG,
                                               const Lane& L) {
    using IO = ChunkIO<F::DK, DV, C, NWF>;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    Pipeline<F::DK, DV, C, NWF> P{lds, seg * Gs, min(NC, seg * Gs + Gs), T, bh * T, false};
    char* lifted = lds + 2 * IO::BUF;              // lifted key tiles of the chunk
    FState<F, DV> st;
    state_zero<W, F, DV>(st);
    P.stage(nullptr, k, v, P.c0, L);
    for (int c = P.c0; c < P.c1; ++c) {
        P.acquire(nullptr, k, v, c, L);            // also: every wavefront is done with chunk c - 1's lifts
        const char* buf = P.buffer(c);
        lift_chunk<F, C, 2, true, false>(nullptr, reinterpret_cast<const bf16_t*>(buf + IO::QB), lifted,
                                         threadIdx.x);
        lds_barrier();
        state_update<W, F, DV, C, 2>(st, lifted, reinterpret_cast<const bf16_t*>(buf + 2 * IO::QB), L);
        compiler_fence();
    }
    constexpr int REC = F::NAT * (DV / 16 + 1) * 256;
    record_store<W, F, DV>(rec + (bh * NSEG + seg) * (size_t)REC, st, L);
}

template <class F, int DV, int C>
constexpr int lds_seg() {
    return 2 * ChunkIO<F::DK, DV, C, NWF>::BUF + 2 * F::NAT * Lifted<C, 2>::TILE;
}

template <class F, int DV, int C>
__global__ __launch_bounds__(64 * NWF) void kata_fact_seg_state(const bf16_t* __restrict__ k,
                                                                const bf16_t* __restrict__ v,
                                                                float* __restrict__ rec, int T,
                                                                int NC, int Gs, int NSEG) {
    __shared__ __attribute__((aligned(16))) char lds[lds_seg<F, DV, C>()];
    const Lane L;
    switch (L.w) {
        case 0: seg_state_body<0, F, DV, C>(k, v, rec, lds, T, NC, Gs, NSEG, as_wave<0>(L)); break;
        case 1: seg_state_body<1, F, DV, C>(k, v, rec, lds, T, NC, Gs, NSEG, as_wave<1>(L)); break;
        case 2: seg_state_body<2, F, DV, C>(k, v, rec, lds, T, NC, Gs, NSEG, as_wave<2>(L)); break;
        default: seg_state_body<3, F, DV, C>(k, v, rec, lds, T, NC, Gs, NSEG, as_wave<3>(L)); break;
    }
}

// ---- output ------------------------------------------------------------------

template <class F, int DV, int C>
constexpr int lds_fwd() {
    return 2 * ChunkIO<F::DK, DV, C, NWF>::BUF + 2 * F::NAT * Lifted<C, 2>::TILE + 2 * Pub<F, DV>::BYTES;
}

template <int W, class F, int DV, int C, bool CAUSAL>
__device__ __forceinline__ void fwd_body(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                         const float* prefix, bf16_t* o, char* lds, int T, int NC,
                                         int Gs, int NSEG, const Lane& L) {
    static_assert(C == 16 * NWF, "one query tile per wavefront");
    using IO = ChunkIO<F::DK, DV, C, NWF>;
    using PB = Pub<F, DV>;
    using Frag = typename std::conditional<F::DK == 16, u32x2_t, u32x4_t>::type;
    constexpr int NTV = DV / 16, NU = NTV + 1;
    constexpr int REC = F::NAT * NU * 256;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    // LDS: published state (hi | lo) | lifted key tiles | two chunk buffers. The
    // published operands come first: the workgroup's LDS starts at address 0,
    // so each operand read is the lane's base plus an immediate offset (an
    // immediate reaches 64 KB), with no address register per read.
    char* pub = lds;
    char* lifted = lds + 2 * PB::BYTES;            // lifted key tiles of the chunk
    Pipeline<F::DK, DV, C, NWF> P{lifted + 2 * F::NAT * Lifted<C, 2>::TILE, seg * Gs,
                                  min(NC, seg * Gs + Gs), T, bh * T, true};
    // the second half of an odd last tile pair is never published: zero it all
    for (int i = threadIdx.x; i < 2 * PB::BYTES / 16; i += 64 * NWF)
        reinterpret_cast<u32x4_t*>(pub)[i] = u32x4_t{0u, 0u, 0u, 0u};

    FState<F, DV> st;
    record_load<W, F, DV>(prefix + (CAUSAL ? bh * NSEG + seg : bh) * (size_t)REC, st, L);
    const u32x4_t ones = ones_op(L);
    const int tt = W;                              // this wavefront's query tile
    const int qrow = 16 * tt + L.c16;

    P.stage(q, k, v, P.c0, L);
    for (int c = P.c0; c < P.c1; ++c) {
        const int n = min(C, T - c * C);
        P.acquire(q, k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bq = reinterpret_cast<const bf16_t*>(buf);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + IO::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * IO::QB);
        // the chunk's lifted queries (and keys, for the state update), and the
        // state before this chunk (the whole sequence's when not causal)
        if constexpr (CAUSAL) lift_chunk<F, C, 2, true, false>(nullptr, bk, lifted, threadIdx.x);
        if (CAUSAL || c == P.c0) {
            publish<W, F, DV>(st, pub, L);
            lds_barrier();
        }

        f32x4_t num[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) num[u] = zero4();
        // ---- inter-chunk term phi(q).S and phi(q).z, split operands; this
        // lane's query features lifted from its row in registers
        {
            float x[F::DK];
            load_row<F::DK>(bq, qrow, x);
            inter_pairs<F, DV>(x, pub, num, L, std::make_integer_sequence<int, F::NPAIR>{});
        }
        // ---- intra-chunk term: weights of keys j <= t of this chunk times [V | 1]
        if constexpr (CAUSAL) {
            const Frag qf = lds_row<2 * F::DK, Frag>(bq, qrow, 2 * L.g * F::EPL);
#pragma unroll
            for (int m = 0; m <= tt / 2; ++m) {
                float w[8];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kb = 2 * m + h;          // 16-key block
                    if (kb > tt) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) w[4 * h + r] = 0.0f;
                        continue;
                    }
                    const f32x4_t sc = weights16<F>(bk, 16 * kb + L.c16, qf, L);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * kb + 4 * L.g + r;
                        w[4 * h + r] = (kb < tt || j <= qrow) ? sc[r] : 0.0f;
                    }
                }
                const u32x4_t a = {pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]), pk2(w[6], w[7])};
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) num[nt] = mma32(v_fragment_tr<DV>(bv, m, nt, L), a, num[nt]);
                num[NTV] = mma32(ones, a, num[NTV]);
            }
        }
        // ---- normalise (0 where the denominator is 0) and store this lane's
        // four columns of each value tile
        const float y = inv_den(__shfl(num[NTV][0], L.c16, 64));
        if (qrow < n) {
            bf16_t* orow = o + (bh * T + (size_t)c * C + qrow) * DV + 4 * L.g;
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
                *reinterpret_cast<u32x2_t*>(orow + 16 * nt) =
                    u32x2_t{pk2(num[nt][0] * y, num[nt][1] * y), pk2(num[nt][2] * y, num[nt][3] * y)};
        }
        // ---- running state (not needed after the segment's last chunk)
        if (CAUSAL && c + 1 < P.c1) state_update<W, F, DV, C, 2>(st, lifted, bv, L);
        compiler_fence();
    }
}

template <class F, int DV, int C, bool CAUSAL>
__global__ __launch_bounds__(64 * NWF) void kata_fact_fwd(const bf16_t* __restrict__ q,
                                                          const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v,
                                                          const float* __restrict__ prefix,
                                                          bf16_t* __restrict__ o, int T, int NC,
                                                          int Gs, int NSEG) {
    __shared__ __attribute__((aligned(16))) char lds[lds_fwd<F, DV, C>()];
    const Lane L;
    switch (L.w) {
        case 0: fwd_body<0, F, DV, C, CAUSAL>(q, k, v, prefix, o, lds, T, NC, Gs, NSEG, as_wave<0>(L)); break;
        case 1: fwd_body<1, F, DV, C, CAUSAL>(q, k, v, prefix, o, lds, T, NC, Gs, NSEG, as_wave<1>(L)); break;
        case 2: fwd_body<2, F, DV, C, CAUSAL>(q, k, v, prefix, o, lds, T, NC, Gs, NSEG, as_wave<2>(L)); break;
        default: fwd_body<3, F, DV, C, CAUSAL>(q, k, v, prefix, o, lds, T, NC, Gs, NSEG, as_wave<3>(L)); break;
    }
}

// ---- record <-> packed (S [D, d_v] row-major, z [D]) -------------------------

__global__ void fact_record_to_packed(const float* __restrict__ rec, float* __restrict__ S,
                                      float* __restrict__ z, int D, int DV, int REC, int nrec) {
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        int a, col;
        bool zt;
        rec1_coords((int)(x % REC), DV / 16, &a, &col, &zt);
        if (a >= D) continue;
        if (!zt) S[(b * D + a) * DV + col] = rec[x];
        else if (col == 0) z[b * D + a] = rec[x];
    }
}

__global__ void fact_record_from_packed(float* __restrict__ rec, const float* __restrict__ S,
                                        const float* __restrict__ z, int D, int DV, int REC,
                                        int nrec) {
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        int a, col;
        bool zt;
        rec1_coords((int)(x % REC), DV / 16, &a, &col, &zt);
        rec[x] = a >= D ? 0.0f : !zt ? S[(b * D + a) * DV + col] : (col == 0 ? z[b * D + a] : 0.0f);
    }
}

// ---- decode step (one block per row, fp32 state in the packed layout) --------

constexpr int kDecThreads = 256;

template <typename TIn, class F, int DV>
__global__ __launch_bounds__(kDecThreads) void fact_decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    float* __restrict__ S, float* __restrict__ z, TIn* __restrict__ o) {
    constexpr int DK = F::DK, D = F::D;
    constexpr int C4 = DV / 4;                     // float4 columns per row
    constexpr int RG = kDecThreads / C4;           // row groups
    constexpr int RPT = (D + RG - 1) / RG;         // rows per thread
    __shared__ float fq[D], fk[D], vs[DV], qs[DK], ks[DK];
    __shared__ float4 red[RG][C4];
    __shared__ float dred[kDecThreads / 64];

    const size_t row = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < DK) {
        qs[tid] = io<TIn>::ld(q, row * DK + tid);
        ks[tid] = io<TIn>::ld(k, row * DK + tid);
    }
    if (tid < DV) vs[tid] = io<TIn>::ld(v, row * DV + tid);
    __syncthreads();
    for (int f = tid; f < D; f += kDecThreads) {
        int a, i, j;
        feature_pair<F>(f, &a, &i, &j);
        const float sc = i == j ? 1.0f : kSqrt2;
        float aq = 0.0f, ak = 0.0f;
#pragma unroll
        for (int b = 0; b < (F::SUMMED ? F::G : 1); ++b) {
            const int base = (F::SUMMED ? b : a) * F::P;
            aq += qs[base + i] * qs[base + j];
            ak += ks[base + i] * ks[base + j];
        }
        fq[f] = sc * aq;
        fk[f] = sc * ak;
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
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int p = rg + u * RG;
        if (p < D) {
            const float a = fk[p], b = fq[p];
            float4 s = cur[u];
            s.x += a * vv.x; s.y += a * vv.y; s.z += a * vv.z; s.w += a * vv.w;
            S4[p * C4 + c4] = s;
            acc.x += b * s.x; acc.y += b * s.y; acc.z += b * s.z; acc.w += b * s.w;
        }
    }
    red[rg][c4] = acc;

    float dpart = 0.0f;
    float* zr = z + row * (size_t)D;
    for (int p = tid; p < D; p += kDecThreads) {
        const float zn = zr[p] + fk[p];
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
        for (int u = 0; u < kDecThreads / 64; ++u) den += dred[u];
        io<TIn>::st(o, row * DV + tid, safe_div(num, den));
    }
}

// ---- dispatch ----------------------------------------------------------------

struct FArgs {
    const void *q, *k, *v;
    float* rec;            // state kernel: segment records
    const float* prefix;   // output kernel: scanned records (causal) or total records
    void* o;
    int causal, Gs, NSEG;
    bool state_only;
};

template <class F, int DV>
hipError_t launch_f_dv(const Shape& s, const FArgs& a, hipStream_t st) {
    constexpr int C = 64;
    dim3 grid(a.NSEG, s.B * s.H);
    const bf16_t *q = (const bf16_t*)a.q, *k = (const bf16_t*)a.k, *v = (const bf16_t*)a.v;
    if (a.state_only)
        kata_fact_seg_state<F, DV, C><<<grid, 64 * NWF, 0, st>>>(k, v, a.rec, s.T, s.NC, a.Gs, a.NSEG);
    else if (a.causal)
        kata_fact_fwd<F, DV, C, true><<<grid, 64 * NWF, 0, st>>>(q, k, v, a.prefix, (bf16_t*)a.o, s.T,
                                                                s.NC, a.Gs, a.NSEG);
    else
        kata_fact_fwd<F, DV, C, false><<<grid, 64 * NWF, 0, st>>>(q, k, v, a.prefix, (bf16_t*)a.o, s.T,
                                                                 s.NC, a.Gs, a.NSEG);
    return hipGetLastError();
}

template <class F>
hipError_t launch_f(const Shape& s, const FArgs& a, hipStream_t st) {
    switch (s.dv) {
        case 32: return launch_f_dv<F, 32>(s, a, st);
        case 64: return launch_f_dv<F, 64>(s, a, st);
    }
    return hipErrorInvalidValue;
}

// Calls fn with the Fact type of (d_k, G, summed); false for an unsupported set.
template <typename Fn>
bool with_fact(int dk, int G, bool summed, Fn&& fn) {
    if (dk == 16 && G == 2) { summed ? fn(Fact<16, 2, true>{}) : fn(Fact<16, 2, false>{}); return true; }
    if (dk == 16 && G == 4) { summed ? fn(Fact<16, 4, true>{}) : fn(Fact<16, 4, false>{}); return true; }
    if (dk == 32 && G == 2 && summed) { fn(Fact<32, 2, true>{}); return true; }
    if (dk == 32 && G == 4) { summed ? fn(Fact<32, 4, true>{}) : fn(Fact<32, 4, false>{}); return true; }
    return false;
}

hipError_t dispatch(const Shape& s, int G, bool summed, const FArgs& a, hipStream_t st) {
    hipError_t e = hipErrorInvalidValue;
    with_fact(s.dk, G, summed, [&](auto f) { e = launch_f<decltype(f)>(s, a, st); });
    return e;
}

unsigned conv_blocks(size_t n) { return (unsigned)std::min<size_t>((n + 255) / 256, 4096); }

template <typename TIn, class F>
hipError_t launch_dec(const void* q, const void* k, const void* v, float* S, float* z, void* o,
                      int N, int dv, hipStream_t st) {
    const TIn *qq = (const TIn*)q, *kk = (const TIn*)k, *vv = (const TIn*)v;
    TIn* oo = (TIn*)o;
    switch (dv) {
        case 16: fact_decode_kernel<TIn, F, 16><<<N, kDecThreads, 0, st>>>(qq, kk, vv, S, z, oo); break;
        case 32: fact_decode_kernel<TIn, F, 32><<<N, kDecThreads, 0, st>>>(qq, kk, vv, S, z, oo); break;
        case 64: fact_decode_kernel<TIn, F, 64><<<N, kDecThreads, 0, st>>>(qq, kk, vv, S, z, oo); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int factored_dim(int dk, int G, bool summed) {
    if (dk <= 0 || G <= 0 || dk % G) return -1;
    const int P = dk / G, NF = P * (P + 1) / 2;
    return summed ? NF : G * NF;
}

bool factored_supported(const Shape& s, int G, bool summed) {
    if (!s.bf16 || s.C != 64 || (s.dv != 32 && s.dv != 64)) return false;
    return with_fact(s.dk, G, summed, [](auto) {});
}

bool factored_decode_supported(int dk, int dv, int G, bool summed) {
    return (dv == 16 || dv == 32 || dv == 64) && with_fact(dk, G, summed, [](auto) {});
}

int factored_record_floats(int dk, int dv, int G, bool summed) {
    const int D = factored_dim(dk, G, summed);
    return D < 0 ? -1 : ((D + 15) / 16) * (dv / 16 + 1) * 256;
}

hipError_t launch_fact_seg_state(const Shape& s, int G, bool summed, const void* k, const void* v,
                                 float* rec, int Gs, int NSEG, hipStream_t st) {
    return dispatch(s, G, summed, FArgs{nullptr, k, v, rec, nullptr, nullptr, 1, Gs, NSEG, true}, st);
}

hipError_t launch_fact_fwd(const Shape& s, int G, bool summed, const void* q, const void* k,
                           const void* v, const float* prefix, void* o, int causal, int Gs,
                           int NSEG, hipStream_t st) {
    return dispatch(s, G, summed, FArgs{q, k, v, nullptr, prefix, o, causal, Gs, NSEG, false}, st);
}

hipError_t launch_fact_record_from_packed(float* rec, const float* S, const float* z, int D,
                                          int dv, int REC, int nrec, hipStream_t st) {
    fact_record_from_packed<<<conv_blocks((size_t)REC * nrec), 256, 0, st>>>(rec, S, z, D, dv, REC, nrec);
    return hipGetLastError();
}

hipError_t launch_fact_record_to_packed(const float* rec, float* S, float* z, int D, int dv,
                                        int REC, int nrec, hipStream_t st) {
    fact_record_to_packed<<<conv_blocks((size_t)REC * nrec), 256, 0, st>>>(rec, S, z, D, dv, REC, nrec);
    return hipGetLastError();
}

hipError_t launch_fact_decode(const void* q, const void* k, const void* v, float* S, float* z,
                              void* o, int N, int dk, int dv, int G, bool summed, bool bf16,
                              hipStream_t st) {
    if (N == 0) return hipSuccess;
    hipError_t e = hipErrorInvalidValue;
    with_fact(dk, G, summed, [&](auto f) {
        e = bf16 ? launch_dec<bf16_t, decltype(f)>(q, k, v, S, z, o, N, dv, st)
                 : launch_dec<float, decltype(f)>(q, k, v, S, z, o, N, dv, st);
    });
    return e;
}

}  // namespace kata
