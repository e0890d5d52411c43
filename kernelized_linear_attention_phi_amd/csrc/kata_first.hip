// First-order (identity feature) chunked forward on gfx950 matrix cores.
//
// The paper's abstract sets an associative scan of the first-order feature's
// inter-chunk recurrence against a matched sequential linear-attention baseline;
// the KATA explainers (gist.science, technical summary 2.2 and 2.3) place the
// first-order feature on the orthant cone and give the recurrence depth as
// O(N_C) sequentially and O(log N_C) with a scan. With phi1(x) = x the weight of
// key j for query t is q_t . k_j, the state is S = sum_j k_j v_j^T (d_k x d_v) and
// z = sum_j k_j, and the output takes the same normalised form as the PSD lift:
// o_t = (A V + q_t P) / (A 1 + q_t Z), zero where the denominator is zero, with
// A = Q K^T masked to j <= t inside the chunk and (P, Z) the state of every
// earlier token.
//
// The same segment / scan / output structure as the PSD kernels, on the same
// staging pipeline. A state record holds accumulator tiles: unit (at, u) of 256
// floats for feature tile at (16 features) and value tile u; u = d_v/16 is the z
// tile, accumulated against the ones operand so that only its column 0 is
// nonzero. Element 4*lane + r of a unit is S[16 at + 4 g + r][16 u + c16].
//
// Decay gate (DECAY, chunk 32 or 64; the same reading as for the PSD lift):
// per chunk the staged log-decays are scanned (lane = position, log2 units);
// key j's K^T fragment entries are scaled by 2^{b_last - b_j} before the state
// update, the state by 2^{b_last}; query t's inter-chunk term by 2^{b_t} and its
// intra weights q_t . k_j by 2^{b_t - b_j}.
//
// Output kernel: two wavefronts; wavefront w owns query tiles w, w + 2, ...
// (causally balanced) and holds the whole state (d_k x d_v is small), so no
// partial sums are exchanged. Wavefront 0 issues every chunk copy and no global
// store; wavefront 1 issues every store (rows staged in LDS by both; wavefront
// 0's in two alternating buffers, since wavefront 1 reads them one chunk later
// while wavefront 0 already stages the next chunk's rows).
#include <algorithm>

#include "kata_chunk.h"
#include "kata_internal.h"
#include "kata_records.h"

namespace kata {

namespace {

constexpr int NW1 = 2;   // wavefronts per workgroup
constexpr int ALL = -1;  // "every unit" in place of a wavefront index

template <int DK, int DV, int C, bool GATE = false>
struct Cfg1 {
    static constexpr int NAT = DK / 16;           // feature tiles
    static constexpr int NTV = DV / 16;           // value tiles
    static constexpr int NU = NTV + 1;            // value tiles and the z tile
    static constexpr int TT = C / 16;             // query tiles per chunk
    static constexpr int TW = TT / NW1;           // query tiles per wavefront
    static constexpr int KS = C / 32;             // 32-token K-steps per chunk
    using IO = ChunkIO<DK, DV, C, NW1, 1, GATE>;
    static constexpr int OROW = DV * 2 + 16;      // LDS row stride of staged output rows
    static constexpr int OST = TW * 16 * OROW;    // staged rows of one wavefront
    // gated: one row of cumulative log-decays per wavefront after the rest
    static constexpr int ROWS = GATE ? NW1 * kKeyDecayRowBytes : 0;
    static constexpr int LDS_FWD = 2 * IO::BUF + 3 * OST + ROWS;   // staged rows: w0 x 2, w1
    static constexpr int NBUF_SEG = 3 * IO::BUF <= 65536 ? 3 : 2;
    static constexpr int LDS_SEG = NBUF_SEG * IO::BUF + ROWS;
    static constexpr int REC = NAT * NU * 256;
    static_assert(TW >= 1 && KS >= 1, "chunk of at least 32 tokens");
};

// Running state: S and z as accumulator tiles, s[at][u].
template <int DK, int DV, int C>
struct State1 {
    f32x4_t s[Cfg1<DK, DV, C>::NAT][Cfg1<DK, DV, C>::NU];
};

// Unit j = at * NU + u of the state: every unit (W == ALL) or those of
// wavefront W (j % NW1 == W).
template <int W, int NU>
__host__ __device__ constexpr bool owns(int at, int u) {
    return W == ALL || (at * NU + u) % NW1 == W;
}

// Value-tile split (the sequential walk): a workgroup of value tile vt
// evaluates only the columns of that tile and the z tile; vt < 0: every tile.
__device__ __forceinline__ bool live_unit(int vt, int u, int NTV) {
    return vt < 0 || u == vt || u == NTV;
}

// The 8 bf16 of an operand fragment, each times its own factor, rounded back.
__device__ __forceinline__ u32x4_t scale_bf16x8(const u32x4_t& x, const float (&f)[8]) {
    u32x4_t y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = pk2(lo_bf16(x[i]) * f[2 * i], hi_bf16(x[i]) * f[2 * i + 1]);
    return y;
}

// The state leaving a chunk: every accumulator times 2^{b_last}.
template <int DK, int DV, int C>
__device__ __forceinline__ void decay_state1(State1<DK, DV, C>& st, const ChunkDecay& cd) {
    const float a = exp2_neg(cd.last);
#pragma unroll
    for (int at = 0; at < Cfg1<DK, DV, C>::NAT; ++at)
#pragma unroll
        for (int u = 0; u < Cfg1<DK, DV, C>::NU; ++u) st.s[at][u] *= a;
}

// S += K_c^T [V_c | 1] over one chunk staged in LDS, for the units wavefront W
// holds: A = K^T fragments (features x tokens), B = V fragments or the ones
// operand (column 0), both read transposed from the row-major chunk.
template <int W, int DK, int DV, int C, bool DECAY = false>
__device__ __forceinline__ void state_update1(State1<DK, DV, C>& st, const bf16_t* bk,
                                              const bf16_t* bv, const Lane& L,
                                              const KeyDecay& kd = KeyDecay{}, int vt = -1) {
    using F = Cfg1<DK, DV, C>;
    const u32x4_t ones = ones_op(L);
#pragma unroll
    for (int m = 0; m < F::KS; ++m) {
        u32x4_t kt[F::NAT];
#pragma unroll
        for (int at = 0; at < F::NAT; ++at) kt[at] = v_fragment_tr<DK>(bk, m, at, L);
        if constexpr (DECAY) {
            // slot s is token 32m + 16(s/4) + 4g + s%4: weight 2^{b_last - b_j}
            float f[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) f[s] = exp2_neg(kd.last - kd.b(2 * m + s / 4, s % 4));
#pragma unroll
            for (int at = 0; at < F::NAT; ++at) kt[at] = scale_bf16x8(kt[at], f);
        }
#pragma unroll
        for (int u = 0; u < F::NU; ++u) {
            if (!live_unit(vt, u, F::NTV)) continue;
            bool any = false;
#pragma unroll
            for (int at = 0; at < F::NAT; ++at) any = any || owns<W, F::NU>(at, u);
            if (!any) continue;
            const u32x4_t b = u < F::NTV ? v_fragment_tr<DV>(bv, m, u, L) : ones;
#pragma unroll
            for (int at = 0; at < F::NAT; ++at)
                if (owns<W, F::NU>(at, u)) st.s[at][u] = mma32(kt[at], b, st.s[at][u]);
        }
    }
}

// Units of a split workgroup: its value tile, and the z tile from value tile 0
// only (every split workgroup of a head holds the same z).
template <int W, int DK, int DV, int C>
__device__ __forceinline__ void record_store1(float* rec, const State1<DK, DV, C>& st,
                                              const Lane& L, int vt = -1) {
    using F = Cfg1<DK, DV, C>;
    f32x4_t* r4 = reinterpret_cast<f32x4_t*>(rec);
#pragma unroll
    for (int at = 0; at < F::NAT; ++at)
#pragma unroll
        for (int u = 0; u < F::NU; ++u)
            if (owns<W, F::NU>(at, u) && live_unit(vt, u, F::NTV) && (u < F::NTV || vt <= 0))
                r4[(at * F::NU + u) * 64 + L.lane] = st.s[at][u];
}

template <int DK, int DV, int C>
__device__ __forceinline__ void record_load1(const float* rec, State1<DK, DV, C>& st,
                                             const Lane& L, int vt = -1) {
    using F = Cfg1<DK, DV, C>;
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(rec);
#pragma unroll
    for (int at = 0; at < F::NAT; ++at)
#pragma unroll
        for (int u = 0; u < F::NU; ++u)
            st.s[at][u] = live_unit(vt, u, F::NTV) ? r4[(at * F::NU + u) * 64 + L.lane] : zero4();
}

// ---- segment states ----------------------------------------------------------

template <int W, int DK, int DV, int C, bool DECAY>
__device__ __forceinline__ void seg_state_body1(const bf16_t* k, const bf16_t* v,
                                                const float* gdec, float* rec, float* segdec,
                                                char* lds, int T, int NC, int G, int NSEG,
                                                const Lane& L) {
    using F = Cfg1<DK, DV, C>;
    using FG = Cfg1<DK, DV, C, DECAY>;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    LoadPipeline<DK, DV, C, NW1, FG::NBUF_SEG, DECAY> P{lds, seg * G, min(NC, seg * G + G), T,
                                                        bh * T, gdec};
    float* krow = reinterpret_cast<float*>(lds + FG::NBUF_SEG * FG::IO::BUF + W * kKeyDecayRowBytes);
    float lsum = 0.0f;                             // log2 of the segment's decay
    State1<DK, DV, C> st;
#pragma unroll
    for (int at = 0; at < F::NAT; ++at)
#pragma unroll
        for (int u = 0; u < F::NU; ++u) st.s[at][u] = zero4();
    P.prologue(k, v, L);
    for (int c = P.c0; c < P.c1; ++c) {
        P.acquire(k, v, c, L);
        const char* buf = P.buffer(c);
        KeyDecay kd{};
        if constexpr (DECAY) {
            const ChunkDecay cd = chunk_decay<C>(buf + 2 * F::IO::QB + F::IO::VB, L);
            kd = key_decays(cd, krow, L);
            decay_state1<DK, DV, C>(st, cd);
            lsum += cd.last;
        }
        state_update1<W, DK, DV, C, DECAY>(st, reinterpret_cast<const bf16_t*>(buf + F::IO::QB),
                                           reinterpret_cast<const bf16_t*>(buf + 2 * F::IO::QB), L,
                                           kd);
        compiler_fence();
    }
    record_store1<W, DK, DV, C>(rec + (bh * NSEG + seg) * (size_t)F::REC, st, L);
    if (DECAY && W == 0 && L.lane == 0) segdec[bh * NSEG + seg] = exp2_neg(lsum);
}

template <int DK, int DV, int C, bool DECAY>
__global__ __launch_bounds__(64 * NW1) void kata_seg_state1(const bf16_t* __restrict__ k,
                                                            const bf16_t* __restrict__ v,
                                                            const float* __restrict__ gdec,
                                                            float* __restrict__ rec,
                                                            float* __restrict__ segdec, int T,
                                                            int NC, int G, int NSEG) {
    __shared__ __attribute__((aligned(16))) char lds[Cfg1<DK, DV, C, DECAY>::LDS_SEG];
    const Lane L;
    if (L.w == 0)
        seg_state_body1<0, DK, DV, C, DECAY>(k, v, gdec, rec, segdec, lds, T, NC, G, NSEG, as_wave<0>(L));
    else
        seg_state_body1<1, DK, DV, C, DECAY>(k, v, gdec, rec, segdec, lds, T, NC, G, NSEG, as_wave<1>(L));
}

// ---- output ------------------------------------------------------------------

// Rows staged by wavefront w (its query tiles NW1*u + w, row stride OROW): staged
// row r goes to oc[16*NW1*(r/16) + r%16] when that is below n (the caller offsets
// oc and n by the wavefront's 16 w rows). Wavefront 1 only.
// SPLIT: only the two 16-byte units of value tile vt of each row.
template <int DK, int DV, int C, bool SPLIT = false>
__device__ __forceinline__ void store_rows1(const char* ost, bf16_t* oc, int n, const Lane& L,
                                            int vt = 0) {
    using F = Cfg1<DK, DV, C>;
    constexpr int UPR = SPLIT ? 2 : DV * 2 / 16;  // 16-byte units stored per row
    constexpr int NUN = F::TW * 16 * UPR;
#pragma unroll
    for (int i = 0; i < (NUN + 63) / 64; ++i) {
        const int unit = L.lane + 64 * i;
        if (unit < NUN) {
            const int rl = unit / UPR, col = (SPLIT ? 2 * vt : 0) + unit % UPR;
            const int row = 16 * NW1 * (rl / 16) + rl % 16;
            const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ost + rl * F::OROW + 16 * col);
            if (row < n) *reinterpret_cast<u32x4_t*>(oc + (size_t)row * DV + 8 * col) = val;
        }
    }
}

// Query fragment of feature tile at for the K = 16 products (B operand: lane c16
// = query row, slots 4g + s = features 16 at + 4g + s).
template <int DK>
__device__ __forceinline__ u32x2_t query16(const bf16_t* bq, int row, int at, const Lane& L) {
    return lds_row<2 * DK, u32x2_t>(bq, row, 32 * at + 8 * L.g);
}

// Scores of 16 keys (rows r .. r+15 of the staged chunk, lane c16 = key r + c16)
// against a query tile: D[key 4g + r'][query c16] = q . k.
template <int DK>
__device__ __forceinline__ f32x4_t scores1(const bf16_t* bk, const bf16_t* bq, int krow, int qrow,
                                           const Lane& L) {
    if constexpr (DK == 16) {
        return mma16(lds_row<32, u32x2_t>(bk, krow, 8 * L.g), lds_row<32, u32x2_t>(bq, qrow, 8 * L.g),
                     zero4());
    } else {
        return mma32(lds_row<64, u32x4_t>(bk, krow, 16 * L.g), lds_row<64, u32x4_t>(bq, qrow, 16 * L.g),
                     zero4());
    }
}

template <int W, int DK, int DV, int C, bool CAUSAL, bool DECAY, bool SPLIT>
__device__ __forceinline__ void fwd_body1(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                          const float* gdec, const float* prefix,
                                          float* final_rec, bf16_t* o, char* lds, int T, int NC,
                                          int G, int NSEG, const Lane& L) {
    using F = Cfg1<DK, DV, C>;
    using FG = Cfg1<DK, DV, C, DECAY>;
    const int seg = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int vt = SPLIT ? (int)blockIdx.z : -1;   // value tile of a split workgroup
    Pipeline<DK, DV, C, NW1, 1, DECAY> P{lds, seg * G, min(NC, seg * G + G), T, bh * T, true, gdec};
    // staged rows: wavefront 0 in buffer (c - c0) % 2, wavefront 1 in buffer 2
    char* ostage = lds + 2 * FG::IO::BUF;
    float* krow = reinterpret_cast<float*>(lds + 2 * FG::IO::BUF + 3 * F::OST + W * kKeyDecayRowBytes);

    State1<DK, DV, C> st;
    record_load1<DK, DV, C>(prefix + (CAUSAL ? bh * NSEG + seg : bh) * (size_t)F::REC, st, L, vt);
    const u32x4_t ones = ones_op(L);

    P.stage(q, k, v, P.c0, L);
    for (int c = P.c0; c < P.c1; ++c) {
        const int n = min(C, T - c * C);
        P.acquire(q, k, v, c, L);
        const char* buf = P.buffer(c);
        const bf16_t* bq = reinterpret_cast<const bf16_t*>(buf);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::IO::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::IO::QB);
        bf16_t* oc = o + (bh * T + (size_t)c * C) * DV;
        // decay gate: the chunk's cumulative log-decays (staged after v)
        ChunkDecay cd{0.0f, 0.0f};
        KeyDecay kd{};
        if constexpr (DECAY) {
            cd = chunk_decay<C>(buf + 2 * F::IO::QB + F::IO::VB, L);
            kd = key_decays(cd, krow, L);
        }

        // wavefront 0's rows of the previous chunk (always a full chunk)
        if (W == 1 && c > P.c0)
            store_rows1<DK, DV, C, SPLIT>(ostage + ((c - 1 - P.c0) & 1) * F::OST,
                                          oc - (size_t)C * DV, C, L, vt);
        compiler_fence();
        char* own = ostage + (W == 0 ? ((c - P.c0) & 1) : 2) * F::OST;

        // the state before this chunk as bf16 A operands of S^T (rows = value
        // columns, K = features); the z tile gives row 0 = z
        u32x2_t sop[F::NAT][F::NU];
#pragma unroll
        for (int at = 0; at < F::NAT; ++at)
#pragma unroll
            for (int u = 0; u < F::NU; ++u)
                sop[at][u] = u32x2_t{pk2(st.s[at][u][0], st.s[at][u][1]),
                                     pk2(st.s[at][u][2], st.s[at][u][3])};

#pragma unroll
        for (int ui = 0; ui < F::TW; ++ui) {
            const int tt = NW1 * ui + W;
            const int qrow = 16 * tt + L.c16;
            // num[u]: D[value 16u + 4g + r][query c16]; num[NTV] row 0 = denominator
            f32x4_t num[F::NU];
#pragma unroll
            for (int u = 0; u < F::NU; ++u) num[u] = zero4();
            // ---- inter-chunk term q.P and q.Z (K = 16 per feature tile)
#pragma unroll
            for (int at = 0; at < F::NAT; ++at) {
                const u32x2_t qa = query16<DK>(bq, qrow, at, L);
#pragma unroll
                for (int u = 0; u < F::NU; ++u)
                    if (live_unit(vt, u, F::NTV)) num[u] = mma16_acc32(sop[at][u], qa, num[u]);
            }
            float bt = 0.0f;                          // b of this lane's query
            if constexpr (DECAY) {                    // the prefix state decays to query t
                bt = krow[qrow];
                const float e = exp2_neg(bt);
#pragma unroll
                for (int u = 0; u < F::NU; ++u) num[u] *= e;
            }
            // ---- intra-chunk term: A = Q K^T masked to j <= t, num += A [V | 1]
            if (CAUSAL) {
#pragma unroll
                for (int m = 0; m <= tt / 2; ++m) {
                    const bool diag = 32 * m + 31 > 16 * tt;
                    float w[8];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f32x4_t sc = scores1<DK>(bk, bq, 32 * m + 16 * h + L.c16, qrow, L);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = 32 * m + 16 * h + 4 * L.g + r;
                            float x = sc[r];
                            if constexpr (DECAY) x *= exp2_neg(bt - kd.b(2 * m + h, r));
                            w[4 * h + r] = (!diag || j <= qrow) ? x : 0.0f;
                        }
                    }
                    const u32x4_t a = {pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]), pk2(w[6], w[7])};
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt)
                        if (live_unit(vt, nt, F::NTV)) num[nt] = mma32(v_fragment_tr<DV>(bv, m, nt, L), a, num[nt]);
                    num[F::NTV] = mma32(ones, a, num[F::NTV]);
                }
            }
            // ---- normalise: o = num / den, den = row 0 of the denominator tile
            const float y = inv_den(__shfl(num[F::NTV][0], L.c16, 64));   // 0 -> o = 0
#pragma unroll
            for (int nt = 0; nt < F::NTV; ++nt)
                if (live_unit(vt, nt, F::NTV))
                    *reinterpret_cast<u32x2_t*>(own + (16 * ui + L.c16) * F::OROW +
                                                2 * (16 * nt + 4 * L.g)) =
                        u32x2_t{pk2(num[nt][0] * y, num[nt][1] * y), pk2(num[nt][2] * y, num[nt][3] * y)};
        }
        // wavefront 1's own rows leave in this chunk, as whole rows
        compiler_fence();
        if (W == 1) store_rows1<DK, DV, C, SPLIT>(own, oc + 16 * DV, n - 16, L, vt);

        // ---- running state: S += K_c^T V_c, z += K_c^T 1 (both wavefronts; not
        // needed after the segment's last chunk unless the final state is asked for)
        if (CAUSAL && (c + 1 < P.c1 || final_rec)) {
            if constexpr (DECAY) decay_state1<DK, DV, C>(st, cd);
            state_update1<ALL, DK, DV, C, DECAY>(st, bk, bv, L, kd, vt);
        }
        compiler_fence();
    }
    // wavefront 0's rows of the last chunk
    lds_barrier();
    if (W == 1) {
        const int cl = P.c1 - 1;
        store_rows1<DK, DV, C, SPLIT>(ostage + ((cl - P.c0) & 1) * F::OST,
                                      o + (bh * T + (size_t)cl * C) * DV, min(C, T - cl * C), L, vt);
    }
    // running state after the segment (the final state when one segment covers
    // the sequence); the two wavefronts hold the same state and split the units
    if (CAUSAL && final_rec) record_store1<W, DK, DV, C>(final_rec + bh * (size_t)F::REC, st, L, vt);
}

template <int DK, int DV, int C, bool CAUSAL, bool DECAY, bool SPLIT = false>
__global__ __launch_bounds__(64 * NW1) void kata_fwd1(const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v,
                                                      const float* __restrict__ gdec,
                                                      const float* __restrict__ prefix,
                                                      float* __restrict__ final_rec,
                                                      bf16_t* __restrict__ o, int T, int NC,
                                                      int G, int NSEG) {
    __shared__ __attribute__((aligned(16))) char lds[Cfg1<DK, DV, C, DECAY>::LDS_FWD];
    const Lane L;
    if (L.w == 0)
        fwd_body1<0, DK, DV, C, CAUSAL, DECAY, SPLIT>(q, k, v, gdec, prefix, final_rec, o, lds, T,
                                                      NC, G, NSEG, as_wave<0>(L));
    else
        fwd_body1<1, DK, DV, C, CAUSAL, DECAY, SPLIT>(q, k, v, gdec, prefix, final_rec, o, lds, T,
                                                      NC, G, NSEG, as_wave<1>(L));
}

// ---- record <-> packed (S [d_k, d_v] row-major, z [d_k]) ---------------------

__global__ void record_to_packed1(const float* __restrict__ rec, float* __restrict__ S,
                                  float* __restrict__ z, int DK, int DV, int REC, int nrec) {
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        int a, col;
        bool zt;
        rec1_coords((int)(x % REC), DV / 16, &a, &col, &zt);
        if (!zt) S[(b * DK + a) * DV + col] = rec[x];
        else if (col == 0) z[b * DK + a] = rec[x];
    }
}

__global__ void record_from_packed1(float* __restrict__ rec, const float* __restrict__ S,
                                    const float* __restrict__ z, int DK, int DV, int REC,
                                    int nrec) {
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < (size_t)REC * nrec;
         x += (size_t)gridDim.x * blockDim.x) {
        const size_t b = x / REC;
        int a, col;
        bool zt;
        rec1_coords((int)(x % REC), DV / 16, &a, &col, &zt);
        rec[x] = !zt ? S[(b * DK + a) * DV + col] : (col == 0 ? z[b * DK + a] : 0.0f);
    }
}

// ---- launchers ---------------------------------------------------------------

// Launch arguments shared by every shape: gdec (log-decays, NULL = no gate;
// causal only, chunk 32 or 64), segdec (per-segment decays, state kernel).
struct Args1 {
    const void *q, *k, *v;
    const float* gdec;
    float* rec;            // state kernel: segment records; output kernel: final_rec
    float* segdec;
    const float* prefix;
    void* o;
    int causal, G, NSEG;
    bool state_only;
    bool split = false;    // causal output: one workgroup per 16-column value tile
};

template <int DK, int DV, int C>
hipError_t launch_dk_dv_c1(const Shape& s, const Args1& a, hipStream_t st) {
    dim3 grid(a.NSEG, s.B * s.H);
    const bf16_t *q = (const bf16_t*)a.q, *k = (const bf16_t*)a.k, *v = (const bf16_t*)a.v;
    bf16_t* o = (bf16_t*)a.o;
    constexpr bool kGate = C == 32 || C == 64;     // gated instantiations
    if (a.gdec && !kGate) return hipErrorInvalidValue;
    if (a.state_only) {
        if constexpr (kGate) {
            if (a.gdec) {
                kata_seg_state1<DK, DV, C, true><<<grid, 64 * NW1, 0, st>>>(k, v, a.gdec, a.rec, a.segdec,
                                                                           s.T, s.NC, a.G, a.NSEG);
                return hipGetLastError();
            }
        }
        kata_seg_state1<DK, DV, C, false><<<grid, 64 * NW1, 0, st>>>(k, v, nullptr, a.rec, nullptr,
                                                                    s.T, s.NC, a.G, a.NSEG);
    } else if (a.causal && a.split) {
        const dim3 sgrid(a.NSEG, s.B * s.H, DV / 16);
        if constexpr (kGate) {
            if (a.gdec) {
                kata_fwd1<DK, DV, C, true, true, true><<<sgrid, 64 * NW1, 0, st>>>(
                    q, k, v, a.gdec, a.prefix, a.rec, o, s.T, s.NC, a.G, a.NSEG);
                return hipGetLastError();
            }
        }
        kata_fwd1<DK, DV, C, true, false, true><<<sgrid, 64 * NW1, 0, st>>>(
            q, k, v, nullptr, a.prefix, a.rec, o, s.T, s.NC, a.G, a.NSEG);
    } else if (a.causal) {
        if constexpr (kGate) {
            if (a.gdec) {
                kata_fwd1<DK, DV, C, true, true><<<grid, 64 * NW1, 0, st>>>(
                    q, k, v, a.gdec, a.prefix, a.rec, o, s.T, s.NC, a.G, a.NSEG);
                return hipGetLastError();
            }
        }
        kata_fwd1<DK, DV, C, true, false><<<grid, 64 * NW1, 0, st>>>(q, k, v, nullptr, a.prefix, a.rec,
                                                                    o, s.T, s.NC, a.G, a.NSEG);
    } else {
        if (a.gdec) return hipErrorInvalidValue;
        kata_fwd1<DK, DV, C, false, false><<<grid, 64 * NW1, 0, st>>>(q, k, v, nullptr, a.prefix, a.rec,
                                                                     o, s.T, s.NC, a.G, a.NSEG);
    }
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dk_dv1(const Shape& s, const Args1& a, hipStream_t st) {
    switch (s.C) {
        case 32: return launch_dk_dv_c1<DK, DV, 32>(s, a, st);
        case 64: return launch_dk_dv_c1<DK, DV, 64>(s, a, st);
        case 128: return launch_dk_dv_c1<DK, DV, 128>(s, a, st);
    }
    return hipErrorInvalidValue;
}

template <int DK>
hipError_t launch_dk1(const Shape& s, const Args1& a, hipStream_t st) {
    switch (s.dv) {
        case 16: return launch_dk_dv1<DK, 16>(s, a, st);
        case 32: return launch_dk_dv1<DK, 32>(s, a, st);
        case 64: return launch_dk_dv1<DK, 64>(s, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch1(const Shape& s, const Args1& a, hipStream_t st) {
    return s.dk == 16 ? launch_dk1<16>(s, a, st) : launch_dk1<32>(s, a, st);
}

unsigned conv_blocks(size_t n) { return (unsigned)std::min<size_t>((n + 255) / 256, 4096); }

}  // namespace

bool first_supported(const Shape& s) {
    return s.bf16 && (s.dk == 16 || s.dk == 32) && (s.dv == 16 || s.dv == 32 || s.dv == 64) &&
           (s.C == 32 || s.C == 64 || s.C == 128);
}

int first_record_floats(int dk, int dv) { return (dk / 16) * (dv / 16 + 1) * 256; }

hipError_t launch_seg_state1(const Shape& s, const void* k, const void* v, float* rec, int G,
                             int NSEG, hipStream_t st) {
    return dispatch1(s, Args1{nullptr, k, v, nullptr, rec, nullptr, nullptr, nullptr, 1, G, NSEG, true}, st);
}

hipError_t launch_fwd1(const Shape& s, const void* q, const void* k, const void* v,
                       const float* prefix, float* final_rec, void* o, int causal, int G,
                       int NSEG, hipStream_t st, bool split) {
    return dispatch1(s, Args1{q, k, v, nullptr, final_rec, nullptr, prefix, o, causal, G, NSEG, false,
                              split && causal}, st);
}

bool first_decay_supported(const Shape& s) { return first_supported(s) && (s.C == 32 || s.C == 64); }

hipError_t launch_seg_state1_decay(const Shape& s, const void* k, const void* v, const float* gdec,
                                   float* rec, float* segdec, int G, int NSEG, hipStream_t st) {
    return dispatch1(s, Args1{nullptr, k, v, gdec, rec, segdec, nullptr, nullptr, 1, G, NSEG, true}, st);
}

hipError_t launch_fwd1_decay(const Shape& s, const void* q, const void* k, const void* v,
                             const float* gdec, const float* prefix, float* final_rec, void* o,
                             int G, int NSEG, hipStream_t st, bool split) {
    return dispatch1(s, Args1{q, k, v, gdec, final_rec, nullptr, prefix, o, 1, G, NSEG, false, split}, st);
}

hipError_t launch_record_from_packed1(float* rec, const float* S, const float* z, int dk, int dv,
                                      int nrec, hipStream_t st) {
    const int REC = first_record_floats(dk, dv);
    record_from_packed1<<<conv_blocks((size_t)REC * nrec), 256, 0, st>>>(rec, S, z, dk, dv, REC, nrec);
    return hipGetLastError();
}

hipError_t launch_record_to_packed1(const float* rec, float* S, float* z, int dk, int dv, int nrec,
                                    hipStream_t st) {
    const int REC = first_record_floats(dk, dv);
    record_to_packed1<<<conv_blocks((size_t)REC * nrec), 256, 0, st>>>(rec, S, z, dk, dv, REC, nrec);
    return hipGetLastError();
}

}  // namespace kata
