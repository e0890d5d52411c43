// Quadratic ("flash-style") bf16 KATA forward on gfx950 matrix cores.
//
// KATA explainers (gist.science, technical summary 2.3 and section 4) and the
// paper's abstract: next to the linear-state chunked form, the attention
// o_t = sum_{j <= t} (q_t . k_j)^2 v_j / sum_{j <= t} (q_t . k_j)^2 can be
// evaluated in its quadratic form by streaming key blocks past a tile of
// queries, as flash attention does. The squared-inner-product weights are
// non-negative polynomials, so no running maximum or rescaling is needed: the
// numerator and the denominator are plain fp32 accumulations, normalised once
// at the end.
//
// One workgroup of four wavefronts owns 16 * FQT * 4 consecutive queries of one
// (batch, head); wavefront w owns FQT consecutive query tiles of 16. Key blocks
// (64 or 128 keys, CfgF) are staged to LDS (k | v, FNBUF buffers, direct-to-LDS
// copies). Per 32-key step: S = K Q^T on MFMA (keys as rows, the query tile as
// columns), A = S^2 in fp32, cast to bf16, then num += V^T A and den += 1^T A on
// MFMA, with V^T fragments read transposed from LDS once per step for all of
// the wavefront's query tiles. A block whose keys all precede the wavefront's
// first query runs as straight-line code with every score product of the block
// issued before the first square, so matrix-core latency is covered by other
// tiles' work; only blocks that reach the diagonal take the per-step path with
// skips and the j <= t mask. The wavefront index is made scalar, so these
// choices are scalar branches rather than lane-masked ones.
//
// Launch order: heaviest query blocks first (causal work grows with the query
// index); when B*H is a multiple of 8, all query blocks of a head go to one of
// the 8 XCDs (dispatch is round-robin over XCDs), so that head's keys and
// values are reused from that XCD's L2.
#include "kata_chunk.h"
#include "kata_internal.h"

namespace kata {

namespace {

#ifndef KATA_FLASH_QT
#define KATA_FLASH_QT 2
#endif
#ifndef KATA_FLASH_NBUF
#define KATA_FLASH_NBUF 2
#endif
#ifndef KATA_FLASH_NW
#define KATA_FLASH_NW 4
#endif

constexpr int FQT = KATA_FLASH_QT;      // query tiles of 16 per wavefront
constexpr int FNW = KATA_FLASH_NW;      // wavefronts per workgroup
constexpr int FQB = 16 * FQT * FNW;     // queries per workgroup
constexpr int FNBUF = KATA_FLASH_NBUF;  // staging depth

// Keys per staged block: 128 halves the barriers per key, and is faster where a
// block's work per wavefront is small (d_k = 32 scores on 16x16x32 products,
// d_v < 64); at d_k = 16, d_v = 64 blocks of 64 measured as fast or faster.
template <int DK, int DV>
struct CfgF {
    static constexpr int FKB = DK == 16 && DV == 64 ? 64 : 128;
    static constexpr int NTV = DV / 16;
    using IO = ChunkIO<DK, DV, FKB, FNW>;
    static constexpr int LDS = FNBUF * IO::BUF;
    static constexpr int KA = DK == 16 ? 4 : 8;   // coordinates per lane in a K-slot group
};

// Query fragment (B operand of K Q^T): lane (c16, g) holds q_t[KA g .. KA g + KA)
// for t = t0 + c16, zero past the end of the sequence.
template <int DK>
struct QFrag {
    u32x4_t x;                                    // d_k = 32: 8 bf16; d_k = 16: first 2 words
};

template <int DK>
__device__ __forceinline__ QFrag<DK> load_qfrag(const bf16_t* qh, int t, int T, const Lane& L) {
    QFrag<DK> f;
    f.x = u32x4_t{0u, 0u, 0u, 0u};
    if (t < T) {
        if constexpr (DK == 32) {
            f.x = *reinterpret_cast<const u32x4_t*>(qh + (size_t)t * DK + 8 * L.g);
        } else {
            const u32x2_t p = *reinterpret_cast<const u32x2_t*>(qh + (size_t)t * DK + 4 * L.g);
            f.x = u32x4_t{p[0], p[1], 0u, 0u};
        }
    }
    return f;
}

// Scores of 16 keys (staged rows r .. r + 15 of the block, lane c16 taking row
// r + c16) against the query tile (columns): D[key 4g + r'][query c16].
template <int DK>
__device__ __forceinline__ f32x4_t key_scores(const bf16_t* bk, int row, const QFrag<DK>& qf,
                                              const Lane& L) {
    if constexpr (DK == 32) {
        const u32x4_t kf = lds_row<2 * DK, u32x4_t>(bk, row, 16 * L.g);
        return mma32(kf, qf.x, zero4());
    } else {
        const u32x2_t kf = lds_row<2 * DK, u32x2_t>(bk, row, 8 * L.g);
        return mma16(kf, u32x2_t{qf.x[0], qf.x[1]}, zero4());
    }
}

// Weights of one 32-key step for a query tile: A = S^2 (fp32) as a bf16 B
// operand (slot 4h + r = key 16h + 4g + r of the step), entries with key j > t
// zeroed when MASK.
template <bool MASK>
__device__ __forceinline__ u32x4_t step_weights(const f32x4_t (&sc)[2], int key0, int t,
                                                const Lane& L) {
    float w[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = sc[h][r] * sc[h][r];
            w[4 * h + r] = (!MASK || key0 + 16 * h + 4 * L.g + r <= t) ? x : 0.0f;
        }
    return u32x4_t{pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]), pk2(w[6], w[7])};
}

// One query block (FQB queries from qb * FQB) of head bh: stream the key blocks
// it needs through LDS, then normalise and store.
template <int DK, int DV, bool CAUSAL>
__device__ __forceinline__ void flash_query_block(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                                  bf16_t* o, int T, int bh, int qb, char* lds,
                                                  const Lane& L) {
    using F = CfgF<DK, DV>;
    constexpr int FKB = F::FKB;
    constexpr int KS = FKB / 32;                  // 32-key steps per staged block
    const size_t head = (size_t)bh * T;
    const int q0 = qb * FQB + 16 * FQT * L.w;    // first query of this wavefront

    QFrag<DK> qf[FQT];
#pragma unroll
    for (int u = 0; u < FQT; ++u) qf[u] = load_qfrag<DK>(q + head * DK, q0 + 16 * u + L.c16, T, L);

    const int nkb = (T + FKB - 1) / FKB;
    const int kb_end = CAUSAL ? min(nkb, (qb * FQB + FQB - 1) / FKB + 1) : nkb;
    LoadPipeline<DK, DV, FKB, FNW, FNBUF> P{lds, 0, kb_end, T, head};

    f32x4_t num[FQT][F::NTV + 1];
#pragma unroll
    for (int u = 0; u < FQT; ++u)
#pragma unroll
        for (int nt = 0; nt <= F::NTV; ++nt) num[u][nt] = zero4();
    const u32x4_t ones = ones_op(L);

    P.prologue(k, v, L);
    for (int kb = 0; kb < kb_end; ++kb) {
        P.acquire(k, v, kb, L);
        const char* buf = P.buffer(kb);
        const bf16_t* bk = reinterpret_cast<const bf16_t*>(buf + F::IO::QB);
        const bf16_t* bv = reinterpret_cast<const bf16_t*>(buf + 2 * F::IO::QB);
        if (!CAUSAL || kb * FKB + FKB - 1 <= q0) {
            // every key of the block precedes every query of this wavefront:
            // straight-line code, all score products issued before the squares
            f32x4_t sc[KS][FQT][2];
#pragma unroll
            for (int m = 0; m < KS; ++m)
#pragma unroll
                for (int u = 0; u < FQT; ++u)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        sc[m][u][h] = key_scores<DK>(bk, 32 * m + 16 * h + L.c16, qf[u], L);
#pragma unroll
            for (int m = 0; m < KS; ++m) {
                u32x4_t vop[F::NTV];
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) vop[nt] = v_fragment_tr<DV>(bv, m, nt, L);
#pragma unroll
                for (int u = 0; u < FQT; ++u) {
                    const u32x4_t at = step_weights<false>(sc[m][u], 0, 0, L);
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) num[u][nt] = mma32(vop[nt], at, num[u][nt]);
                    num[u][F::NTV] = mma32(ones, at, num[u][F::NTV]);
                }
            }
        } else {
            // the block reaches past the first query of this wavefront: steps
            // after every own query are skipped, tiles whose queries all precede
            // the step too, and steps crossing a tile's diagonal are masked
#pragma unroll
            for (int m = 0; m < KS; ++m) {
                const int key0 = kb * FKB + 32 * m;
                if (key0 > q0 + 16 * FQT - 1) continue;
                u32x4_t vop[F::NTV];
#pragma unroll
                for (int nt = 0; nt < F::NTV; ++nt) vop[nt] = v_fragment_tr<DV>(bv, m, nt, L);
#pragma unroll
                for (int u = 0; u < FQT; ++u) {
                    const int t0 = q0 + 16 * u;
                    if (key0 > t0 + 15) continue;
                    f32x4_t sc[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        sc[h] = key_scores<DK>(bk, 32 * m + 16 * h + L.c16, qf[u], L);
                    const u32x4_t at = key0 + 31 > t0 ? step_weights<true>(sc, key0, t0 + L.c16, L)
                                                      : step_weights<false>(sc, key0, 0, L);
#pragma unroll
                    for (int nt = 0; nt < F::NTV; ++nt) num[u][nt] = mma32(vop[nt], at, num[u][nt]);
                    num[u][F::NTV] = mma32(ones, at, num[u][F::NTV]);
                }
            }
        }
        compiler_fence();
    }

    // ---- normalise and store: o = num / den (den = 0 -> o = 0)
#pragma unroll
    for (int u = 0; u < FQT; ++u) {
        const int t = q0 + 16 * u + L.c16;
        const float den = __shfl(num[u][F::NTV][0], L.c16, 64);
        const float y = inv_den(den);   // y = 0 gives o = 0
#pragma unroll
        for (int nt = 0; nt < F::NTV; ++nt) {
            float ov[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ov[r] = num[u][nt][r] * y;
            }
            if (t < T)
                *reinterpret_cast<u32x2_t*>(o + (head + t) * DV + 16 * nt + 4 * L.g) =
                    u32x2_t{pk2(ov[0], ov[1]), pk2(ov[2], ov[3])};
        }
    }
}

template <int DK, int DV, bool CAUSAL>
__global__ __launch_bounds__(64 * FNW) void kata_flash_fwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ o, int T, int NQB, int BH) {
    __shared__ __attribute__((aligned(16))) char lds[CfgF<DK, DV>::LDS];
    Lane L;
    // the wavefront index is uniform: as a scalar, every per-wavefront condition
    // (causal skips, the masked diagonal path) is a scalar branch
    L.w = __builtin_amdgcn_readfirstlane(L.w);
    // block -> (head, query block), heaviest first, head-to-XCD affinity
    const int lin = blockIdx.x;
    int bh, qb;
    if (BH % 8 == 0) {
        const int xcd = lin % 8, slot = lin / 8, hpx = BH / 8;
        qb = NQB - 1 - slot / hpx;
        bh = (slot % hpx) * 8 + xcd;
    } else {
        qb = NQB - 1 - lin / BH;
        bh = lin % BH;
    }
    flash_query_block<DK, DV, CAUSAL>(q, k, v, o, T, bh, qb, lds, L);
}

template <int DK, int DV>
hipError_t launch_flash_dk_dv(const Shape& s, const void* q, const void* k, const void* v,
                              void* o, bool causal, hipStream_t st) {
    const int BH = s.B * s.H;
    const int NQB = (s.T + FQB - 1) / FQB;
    const unsigned blocks = (unsigned)NQB * BH;
    if (causal)
        kata_flash_fwd_kernel<DK, DV, true><<<blocks, 64 * FNW, 0, st>>>(
            (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)o, s.T, NQB, BH);
    else
        kata_flash_fwd_kernel<DK, DV, false><<<blocks, 64 * FNW, 0, st>>>(
            (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)o, s.T, NQB, BH);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_flash_dk(const Shape& s, const void* q, const void* k, const void* v, void* o,
                           bool causal, hipStream_t st) {
    switch (s.dv) {
        case 16: return launch_flash_dk_dv<DK, 16>(s, q, k, v, o, causal, st);
        case 32: return launch_flash_dk_dv<DK, 32>(s, q, k, v, o, causal, st);
        case 64: return launch_flash_dk_dv<DK, 64>(s, q, k, v, o, causal, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool flash_supported(const Shape& s) {
    return s.bf16 && (s.dk == 16 || s.dk == 32) && (s.dv == 16 || s.dv == 32 || s.dv == 64);
}

hipError_t launch_flash_fwd(const Shape& s, const void* q, const void* k, const void* v, void* o,
                            int causal, hipStream_t st) {
    if ((size_t)s.B * s.H * ((s.T + FQB - 1) / FQB) > 0x7fffffff) return hipErrorInvalidValue;
    return s.dk == 16 ? launch_flash_dk<16>(s, q, k, v, o, causal != 0, st)
                      : launch_flash_dk<32>(s, q, k, v, o, causal != 0, st);
}

}  // namespace kata
