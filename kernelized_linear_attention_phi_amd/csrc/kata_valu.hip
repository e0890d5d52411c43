// fp32 chunked-state path: every product and sum in fp32. Chunk states
// phi(K)^T V run on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: fp32
// operands, fp32 accumulation), everything else on the vector ALUs. It serves
// fp32 inputs (whose tolerance a bf16 matrix-core operand would exceed) and
// stands as the general-shape path.
//
// Chunked-state form (KATA explainers, gist.science, technical summary 2.3):
// chunk c covers positions [cC, min(cC+C, T)); its output is the masked
// intra-chunk term plus phi(Q_c) times the exclusive prefix of chunk states.
//
// Feature (ident): the PSD lift phi(x) (packed pairs, sqrt(2) off the
// diagonal, weight (q.k)^2) or the first-order identity phi1(x) = x (state
// d_k x d_v, weight q.k).
//
// Decay gate (gdec != NULL): per-token log-decays g <= 0 scale the state
// before each token is added (gated linear recurrences, KATA explainers,
// technical summary 1). With b_t = g_0 + ... + g_t inside the chunk (summed in
// float64, so that differences stay accurate after a very negative gate), the
// chunk state weights token j by exp(b_last - b_j) and leaves with the factor
// exp(b_last) for the scan; query t sees the prefix state scaled by exp(b_t)
// and key j <= t of its own chunk by exp(b_t - b_j).
#include "kata_device.h"
#include "kata_internal.h"
#include "kata_mfma.h"

namespace kata {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxC = 128;
constexpr int kMaxDk = 32;
constexpr int kMaxDv = 64;
constexpr int kMaxD = kMaxDk * (kMaxDk + 1) / 2;

// Inclusive sum of the chunk's log-decays in float64: bs[t] = g_0 + ... + g_t
// for t < n (one thread; at most 128 terms).
__device__ __forceinline__ void chunk_log_decay(const float* g, int n, double* bs) {
    if (threadIdx.x == 0) {
        double acc = 0.0;
        for (int t = 0; t < n; ++t) {
            acc += (double)g[t];
            bs[t] = acc;
        }
    }
}

// Copies `count` contiguous inputs (a multiple of 16 bytes' worth, from a
// 16-byte aligned address) to fp32 in LDS: every thread issues all of its
// 16-byte loads before it converts and stores any of them, so the block waits
// about one memory latency rather than one per element.
template <typename TIn, int MAXCOUNT>
__device__ __forceinline__ void stage_f32(const TIn* __restrict__ src, int count, float* dst) {
    constexpr int EPU = 16 / (int)sizeof(TIn);              // elements per 16-byte unit
    constexpr int MAXU = (MAXCOUNT / EPU + kThreads - 1) / kThreads;
    const int units = count / EPU;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4 buf[MAXU];
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const int idx = threadIdx.x + u * kThreads;
        if (idx < units) buf[u] = s4[idx];
    }
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const int idx = threadIdx.x + u * kThreads;
        if (idx >= units) continue;
        const uint32_t wv[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
        if constexpr (sizeof(TIn) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[idx * 8 + 2 * e] = __uint_as_float(wv[e] << 16);
                dst[idx * 8 + 2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[idx * 4 + e] = __uint_as_float(wv[e]);
        }
    }
}

// Copies `count` contiguous inputs (16-byte units from a 16-byte aligned
// address) to LDS unchanged, all loads in flight before the first store.
template <typename TIn, int MAXCOUNT>
__device__ __forceinline__ void stage_raw(const TIn* __restrict__ src, int count, TIn* dst) {
    constexpr int EPU = 16 / (int)sizeof(TIn);
    constexpr int MAXU = (MAXCOUNT / EPU + kThreads - 1) / kThreads;
    const int units = count / EPU;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    uint4 buf[MAXU];
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const int idx = threadIdx.x + u * kThreads;
        if (idx < units) buf[u] = s4[idx];
    }
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const int idx = threadIdx.x + u * kThreads;
        if (idx < units) d4[idx] = buf[u];
    }
}

// S_c = phi(K_c)^T V_c, z_c = phi(K_c)^T 1 for one (head, chunk) per block.
// With the gate, token j is weighted exp(b_last - b_j) and cdec receives the
// chunk's factor exp(b_last). S on the fp32 matrix cores: wavefront w takes
// feature tiles w, w + 4, ... (16 features each, the last one partial); per
// 4-token K-step lane l lifts phi(K)^T[16 ft + l % 16][4 s + l / 16] in fp32 (A)
// and loads V[4 s + l / 16][16 nt + l % 16] (B) for each 16-column value tile;
// the result holds S[16 ft + 4 (l / 16) + r][16 nt + l % 16] in slot r.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void chunk_states_valu(
    const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ gdec,
    float* __restrict__ S_rec, float* __restrict__ z_rec, float* __restrict__ cdec, int T, int dk,
    int dv, int C, int NC, int ident) {
    // LDS sized for this shape (chunk_states_lds): bs | ks | vs | wt | pairs,
    // k and v kept in the input type and widened to fp32 (exactly) when read
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int D = ident ? dk : dk * (dk + 1) / 2;
    double* bs = reinterpret_cast<double*>(smem);
    TIn* ks = reinterpret_cast<TIn*>(smem + C * 8);
    TIn* vs = ks + C * dk;
    float* wt = reinterpret_cast<float*>(vs + C * dv);
    uint32_t* pairs = reinterpret_cast<uint32_t*>(wt + C);
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const TIn* kb = k + (bh * T + t0) * dk;
    const TIn* vb = v + (bh * T + t0) * dv;
    stage_raw<TIn, kMaxC * kMaxDk>(kb, n * dk, ks);
    stage_raw<TIn, kMaxC * kMaxDv>(vb, n * dv, vs);
    fill_pair_table(pairs, dk, D);
    if (gdec) chunk_log_decay(gdec + bh * T + t0, n, bs);
    __syncthreads();
    const size_t rec = bh * NC + c;
    if (gdec) {
        for (int t = threadIdx.x; t < n; t += kThreads) wt[t] = expf((float)(bs[n - 1] - bs[t]));
        if (threadIdx.x == 0) cdec[rec] = expf((float)bs[n - 1]);
        __syncthreads();
    }
    float* Sr = S_rec + rec * D * dv;
    float* zr = z_rec + rec * D;
    // S on the matrix cores (see above); 4 wavefronts of 64 lanes
    static_assert(kThreads == 256, "four wavefronts");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const int nft = (D + 15) / 16, ntv = dv / 16, nks = (n + 3) / 4;
    for (int ft = w; ft < nft; ft += 4) {
        const int p = 16 * ft + r16;                 // this lane's feature (A row)
        const bool live = p < D;
        const int i = !live ? 0 : ident ? p : pairs[p] & 0xff;
        const int j = !live ? 0 : ident ? p : pairs[p] >> 8;
        const float sc = i == j ? 1.0f : kSqrt2;
        f32x4_t acc[kMaxDv / 16];
#pragma unroll
        for (int nt = 0; nt < kMaxDv / 16; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float zacc = 0.0f;                           // z[p] over this lane's tokens
        for (int st = 0; st < nks; ++st) {
            const int t = 4 * st + kq;               // this lane's token (A column, B row)
            float a = 0.0f;
            if (live && t < n) {
                const float ki = io<TIn>::ld(ks, t * dk + i);
                a = ident ? ki : sc * (ki * io<TIn>::ld(ks, t * dk + j));
                if (gdec) a *= wt[t];
            }
            zacc += a;
#pragma unroll
            for (int nt = 0; nt < kMaxDv / 16; ++nt) {
                if (nt >= ntv) break;
                const float b = t < n ? io<TIn>::ld(vs, t * dv + 16 * nt + r16) : 0.0f;
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[nt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int nt = 0; nt < kMaxDv / 16; ++nt) {
            if (nt >= ntv) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pf = 16 * ft + 4 * kq + r;
                if (pf < D) Sr[(size_t)pf * dv + 16 * nt + r16] = acc[nt][r];
            }
        }
        // z[p]: the four lane groups hold the tokens of each residue mod 4
        zacc += __shfl_xor(zacc, 16, 64);
        zacc += __shfl_xor(zacc, 32, 64);
        if (kq == 0 && live) zr[p] = zacc;
    }
}

// Bytes of LDS chunk_states_valu uses for a shape (its layout above); esize
// is the input element size.
size_t chunk_states_lds(int dk, int dv, int C, int D, int esize) {
    return (size_t)C * 8 + (size_t)C * dk * esize + (size_t)C * dv * esize + (size_t)C * 4 +
           (size_t)D * 4;
}

// o for one (head, chunk): inter term phi(q_t).P_c plus the intra term over the
// chunk's positions j <= t, normalised. Non-causal: P is the total state of the
// head and there is no intra term.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void fwd_valu(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ gdec, const float* __restrict__ S_rec,
    const float* __restrict__ z_rec, TIn* __restrict__ o, int T, int dk, int dv, int C, int NC,
    int causal, int ident) {
    __shared__ float qs[kMaxC * kMaxDk];
    __shared__ float ks[kMaxC * kMaxDk];
    __shared__ float vs[kMaxC * kMaxDv];
    __shared__ uint32_t pairs[kMaxD];
    __shared__ double bs[kMaxC];
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int D = ident ? dk : dk * (dk + 1) / 2;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const TIn* qb = q + (bh * T + t0) * dk;
    const TIn* kb = k + (bh * T + t0) * dk;
    const TIn* vb = v + (bh * T + t0) * dv;
    stage_f32<TIn, kMaxC * kMaxDk>(qb, n * dk, qs);
    stage_f32<TIn, kMaxC * kMaxDk>(kb, n * dk, ks);
    stage_f32<TIn, kMaxC * kMaxDv>(vb, n * dv, vs);
    fill_pair_table(pairs, dk, D);
    if (gdec) chunk_log_decay(gdec + bh * T + t0, n, bs);
    __syncthreads();

    const size_t rec = causal ? bh * NC + c : bh;
    const float* P = S_rec + rec * D * dv;
    const float* Z = z_rec + rec * D;
    const int tpc = kThreads / C;              // threads per position
    const int t = threadIdx.x / tpc;
    const int g = threadIdx.x % tpc;
    if (t >= n) return;
    constexpr int kMaxCols = kMaxDv;           // dv / tpc <= 32 for C <= 128
    float num[kMaxCols / 2];
    const int ncols = (dv + tpc - 1) / tpc;
#pragma unroll
    for (int u = 0; u < kMaxCols / 2; ++u) num[u] = 0.0f;
    float den = 0.0f;
    const float* qt = qs + t * dk;
    for (int p = 0; p < D; ++p) {
        const int i = ident ? p : pairs[p] & 0xff, j = ident ? p : pairs[p] >> 8;
        const float fq = ident ? qt[i] : (i == j ? 1.0f : kSqrt2) * (qt[i] * qt[j]);
        den += fq * Z[p];
#pragma unroll
        for (int u = 0; u < kMaxCols / 2; ++u)
            if (u < ncols && g + u * tpc < dv) num[u] += fq * P[p * dv + g + u * tpc];
    }
    if (gdec) {                                // the prefix state decays to query t
        const float e = expf((float)bs[t]);
        den *= e;
#pragma unroll
        for (int u = 0; u < kMaxCols / 2; ++u) num[u] *= e;
    }
    if (causal) {
        for (int jj = 0; jj <= t; ++jj) {
            float s = 0.0f;
            for (int i = 0; i < dk; ++i) s += qt[i] * ks[jj * dk + i];
            float w = ident ? s : s * s;
            if (gdec) w *= expf((float)(bs[t] - bs[jj]));
            den += w;
#pragma unroll
            for (int u = 0; u < kMaxCols / 2; ++u)
                if (u < ncols && g + u * tpc < dv) num[u] += w * vs[jj * dv + g + u * tpc];
        }
    }
    TIn* ob = o + (bh * T + t0 + t) * dv;
#pragma unroll
    for (int u = 0; u < kMaxCols / 2; ++u)
        if (u < ncols && g + u * tpc < dv) io<TIn>::st(ob, g + u * tpc, safe_div(num[u], den));
}

}  // namespace

hipError_t launch_chunk_states_valu(const Shape& s, const void* k, const void* v,
                                    const float* gdec, float* S_rec, float* z_rec, float* cdec,
                                    int ident, hipStream_t st) {
    dim3 grid(s.NC, s.B * s.H);
    const size_t lds = chunk_states_lds(s.dk, s.dv, s.C, ident ? s.dk : s.dk * (s.dk + 1) / 2,
                                        s.bf16 ? 2 : 4);
    if (s.bf16)
        chunk_states_valu<bf16_t><<<grid, kThreads, lds, st>>>(
            (const bf16_t*)k, (const bf16_t*)v, gdec, S_rec, z_rec, cdec, s.T, s.dk, s.dv, s.C,
            s.NC, ident);
    else
        chunk_states_valu<float><<<grid, kThreads, lds, st>>>(
            (const float*)k, (const float*)v, gdec, S_rec, z_rec, cdec, s.T, s.dk, s.dv, s.C,
            s.NC, ident);
    return hipGetLastError();
}

hipError_t launch_fwd_valu(const Shape& s, const void* q, const void* k, const void* v,
                           const float* gdec, const float* S_rec, const float* z_rec, void* o,
                           int causal, int ident, hipStream_t st) {
    dim3 grid(s.NC, s.B * s.H);
    if (s.bf16)
        fwd_valu<bf16_t><<<grid, kThreads, 0, st>>>(
            (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, gdec, S_rec, z_rec,
            (bf16_t*)o, s.T, s.dk, s.dv, s.C, s.NC, causal, ident);
    else
        fwd_valu<float><<<grid, kThreads, 0, st>>>(
            (const float*)q, (const float*)k, (const float*)v, gdec, S_rec, z_rec, (float*)o,
            s.T, s.dk, s.dv, s.C, s.NC, causal, ident);
    return hipGetLastError();
}

}  // namespace kata
