// Pieces shared by the matrix-core chunked-forward kernels (d_k = 16 and 32):
// lane coordinates, constant MFMA operands, the workgroup barrier, LDS
// transposed reads, and the direct-to-LDS staging of one chunk of q | k | v.
//
// Chunks (KATA explainers, gist.science, technical summary 2.3): chunk c of a
// sequence covers positions [cC, min(cC + C, T)); a ragged last chunk is staged
// with zero rows past the end, which add nothing to any sum.
#pragma once

#include "kata_device.h"
#include "kata_mfma.h"

namespace kata {

struct Lane {
    int lane, c16, g, w;
    __device__ Lane()
        : lane(threadIdx.x & 63), c16(threadIdx.x & 15), g((threadIdx.x >> 4) & 3),
          w(threadIdx.x >> 6) {}
};

// The same lane with its wavefront index as a compile-time constant, for a body
// specialised to wavefront W: work selected by wavefront (which chunk pieces it
// copies, which rows it stores) then folds to straight-line code instead of
// lane-masked branches, and no per-piece address stays live for other
// wavefronts' pieces.
template <int W>
__device__ __forceinline__ Lane as_wave(const Lane& L) {
    Lane x = L;
    x.w = W;
    return x;
}

// Row (or column) 0 of the "ones" operand = 1 on every K-slot: as the A operand
// of A.V it turns row 0 of the product into the column sums of the B operand.
__device__ __forceinline__ u32x4_t ones_op(const Lane& L) {
    const uint32_t x = L.c16 == 0 ? 0x3f803f80u : 0u;   // bf16 1.0 twice
    return u32x4_t{x, x, x, x};
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

// Workgroup barrier that waits only for this wavefront's LDS operations (not for
// its outstanding global loads, which may be prefetches).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0), other counters free
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Reciprocal of a denominator for a bf16 output row: v_rcp_f32 (within 1 ulp),
// and 0 for den == 0 so that the row's output is 0. o = num * y is then within
// 2 fp32 ulps of num / den; rounding to bf16 (8 bits of mantissa) takes the same
// value as for the correctly rounded quotient except within 2 fp32 ulps of a
// bf16 rounding midpoint.
__device__ __forceinline__ float inv_den(float den) {
    return den != 0.0f ? __builtin_amdgcn_rcpf(den) : 0.0f;
}

// 16-byte global store at base + off (base wavefront-uniform, off the lane's
// 32-bit byte offset): the address is formed as scalar base plus a 32-bit
// offset, so no 64-bit per-lane address has to stay live.
__device__ __forceinline__ void store16(void* base, uint32_t off, const u32x4_t& val) {
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(base) + (size_t)off) = val;
}

// Value of lane (c16 + d) mod 16 of the same row, for a compile-time d.
template <int D>
__device__ __forceinline__ float partner(float x) {
    if constexpr (D == 0) return x;
    else return row_fetch<D>(x);
}

// Staged rows (q, k, v of a chunk in LDS) are stored XOR-swizzled in 16-byte
// units: unit c of row r sits at unit c ^ swz(r) of that row, with
// swz(r) = (r / (16 / U)) & (U - 1) for U units per row. The 16 consecutive rows
// a group of lanes reads at one column then fall on 16 distinct 16-byte slots
// of the 64 four-byte banks instead of 2 to 8 of them. The swizzle is its own
// inverse within a row, so the same map gives the slot of a unit and the unit of
// a slot.
template <int ROWB>
struct Swz {
    static_assert(ROWB == 32 || ROWB == 64 || ROWB == 128, "row of 2, 4 or 8 units");
    static constexpr int U = ROWB / 16;          // 16-byte units per row
    static constexpr int RPB = 16 / U;           // rows per 256-byte span of the banks
    __host__ __device__ static constexpr int swz(int r) { return (r / RPB) & (U - 1); }
    // LDS byte offset of byte b of row r
    __host__ __device__ static constexpr int off(int r, int b) {
        return r * ROWB + (((b >> 4) ^ swz(r)) << 4) + (b & 15);
    }
    // unit index <-> slot index (an involution)
    __host__ __device__ static constexpr int slot(int u) {
        return (u / U) * U + ((u % U) ^ swz(u / U));
    }
};

// Element read of a staged row: byte b of row r of the buffer at base.
template <int ROWB, typename T>
__device__ __forceinline__ T lds_row(const bf16_t* base, int r, int b) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + Swz<ROWB>::off(r, b));
}

// ds_read_b64_tr_b16: every lane supplies the LDS address of 4 consecutive
// 16-bit elements; within each group of 16 lanes, lane l receives element l % 4
// of the block of lane 4i + l / 4 as its element i (i = 0..3).
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
    const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, r);
}

// V^T fragment of the 32-token K-step m and value tile nt, read transposed from
// the staged [C][DV] chunk in LDS: lane (c16, g), slot s holds
// v[32m + 16(s/4) + 4g + s%4][16nt + c16]. Lane j of group g points at row
// 32m + 16h + 4g + j/4, columns 16nt + 4(j%4) .. +3.
template <int DV>
__device__ __forceinline__ u32x4_t v_fragment_tr(const bf16_t* bv, int m, int nt, const Lane& L) {
    u32x2_t h2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        h2[h] = lds_read_tr16(reinterpret_cast<const char*>(bv) +
                              Swz<2 * DV>::off(32 * m + 16 * h + 4 * L.g + (L.c16 >> 2),
                                               32 * nt + 8 * (L.c16 & 3)));
    return u32x4_t{h2[0][0], h2[0][1], h2[1][0], h2[1][1]};
}

// Direct-to-LDS copy of 16 bytes per lane: lane l moves 16 bytes from gsrc (its
// own address) to LDS lds_dst + 16 l (lds_dst wavefront-uniform, through M0).
// Issued as inline assembly so that the compiler does not track it: with more
// than eight such loads in flight it would otherwise make every later LDS read
// wait for all of them, which serialises the one-chunk-ahead prefetch. Every
// read of a staged buffer is ordered by the pipeline's own vmcnt wait and
// barrier instead. The leading s_nop is the wait state between the M0 write the
// compiler places before the statement and the DMA that reads M0. The address
// stays a per-lane 64-bit vector operand: a scalar base would have to be
// written by v_readfirstlane where the compiler holds it in vector registers,
// and a vector-ALU write of a scalar register needs more wait states before a
// memory instruction reads it than the compiler's hazard check gives an
// inline-assembly operand.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_dst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(lds_dst) : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p);
}

// ---- chunk staging: q | k | v (| g) of one chunk, row-major as in HBM --------
// Full chunks are loaded by the first NLOAD wavefronts only (a wavefront that
// issues no loads never waits for its own stores when it waits for data).
// GATE adds the chunk's C per-token log-decays (fp32) after v; wavefront 0
// copies them before any other piece.
template <int DK, int DV, int C, int NW, int NLOAD = NW, bool GATE = false>
struct ChunkIO {
    static constexpr int QB = C * DK * 2;         // bytes of a q or k chunk
    static constexpr int VB = C * DV * 2;         // bytes of a v chunk
    static constexpr int GB = GATE ? C * 4 : 0;   // bytes of the log-decays
    static constexpr int BUF = 2 * QB + VB + GB;  // one chunk buffer
    static_assert(QB % 1024 == 0 && VB % 1024 == 0, "chunks are whole 1 KB pieces");
    static_assert(GB <= 1024, "the log-decays fit one partial piece");

    // Full chunk: the 1 KB pieces are split round-robin over the loading
    // wavefronts; piece i goes to wavefront i % NLOAD as a direct-to-LDS load.
    // Lane l fills 16-byte slot l of the piece with the unit the swizzle puts
    // there.
    static __device__ __forceinline__ void stage_async(const bf16_t* q, const bf16_t* k,
                                                       const bf16_t* v, const float* gate,
                                                       size_t tok0, uint32_t buf_lds,
                                                       bool with_q, const Lane& L) {
        const char* gq = reinterpret_cast<const char*>(q + tok0 * DK);
        const char* gk = reinterpret_cast<const char*>(k + tok0 * DK);
        const char* gv = reinterpret_cast<const char*>(v + tok0 * DV);
        constexpr int PQ = QB / 1024, PV = VB / 1024;
        const int lane = L.lane;
        if constexpr (GATE) {
            if (L.w == 0 && lane < GB / 16) dma16(gate + tok0 + 4 * lane, buf_lds + 2 * QB + VB);
        }
        const int first = with_q ? 0 : PQ;
#pragma unroll
        for (int i = 0; i < 2 * PQ + PV; ++i) {
            if (i < first || i % NLOAD != L.w) continue;
            const char* src = i < PQ ? gq + 16 * Swz<2 * DK>::slot(64 * i + lane)
                            : i < 2 * PQ ? gk + 16 * Swz<2 * DK>::slot(64 * (i - PQ) + lane)
                                         : gv + 16 * Swz<2 * DV>::slot(64 * (i - 2 * PQ) + lane);
            dma16(src, buf_lds + i * 1024);
        }
    }

    // Ragged chunk (n < C valid positions): bounded loads, zero fill, then LDS.
    static __device__ __forceinline__ void stage_ragged(const bf16_t* q, const bf16_t* k,
                                                        const bf16_t* v, const float* gate,
                                                        size_t tok0, int n, char* buf,
                                                        bool with_q, const Lane& L) {
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        const u32x4_t* gq = reinterpret_cast<const u32x4_t*>(q + tok0 * DK);
        const u32x4_t* gk = reinterpret_cast<const u32x4_t*>(k + tok0 * DK);
        const u32x4_t* gv = reinterpret_cast<const u32x4_t*>(v + tok0 * DV);
        u32x4_t* lq = reinterpret_cast<u32x4_t*>(buf);
        u32x4_t* lk = reinterpret_cast<u32x4_t*>(buf + QB);
        u32x4_t* lv = reinterpret_cast<u32x4_t*>(buf + 2 * QB);
        constexpr int QU = QB / 16, VU = VB / 16;       // 16-byte units
        constexpr int QPR = DK * 2 / 16, VPR = DV * 2 / 16;   // units per row
        const int tid = L.w * 64 + L.lane, nthr = NW * 64;
        for (int u = tid; u < QU; u += nthr) {
            const bool ok = u / QPR < n;
            const int sl = Swz<2 * DK>::slot(u);
            if (with_q) lq[sl] = ok ? gq[u] : zero;
            lk[sl] = ok ? gk[u] : zero;
        }
        for (int u = tid; u < VU; u += nthr) lv[Swz<2 * DV>::slot(u)] = (u / VPR < n) ? gv[u] : zero;
        if constexpr (GATE) {
            float* lg = reinterpret_cast<float*>(buf + 2 * QB + VB);
            for (int t = tid; t < C; t += nthr) lg[t] = t < n ? gate[tok0 + t] : 0.0f;
        }
        compiler_fence();
    }

    // Copies wavefront w issues for one full chunk: every piece from `first` on
    // (its share), plus the log-decays for wavefront 0.
    static __host__ __device__ constexpr int issued(int w, int first) {
        int n = GATE && w == 0 ? 1 : 0;
        for (int i = first; i < 2 * (QB / 1024) + VB / 1024; ++i) n += (i % NLOAD == w);
        return n;
    }
    // Its k and v pieces only (they follow its log-decay and q copies).
    static __host__ __device__ constexpr int kv_pieces(int w) {
        int n = 0;
        for (int i = QB / 1024; i < 2 * (QB / 1024) + VB / 1024; ++i) n += (i % NLOAD == w);
        return n;
    }
};

// vmcnt(n) for a run-time n in 0..15 (larger n waits for everything).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    switch (n) {
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 13: wait_vmcnt<13>(); break;
        case 14: wait_vmcnt<14>(); break;
        case 15: wait_vmcnt<15>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// ---- decay gate: per-chunk cumulative log-decays ----------------------------
// Per-token log-decays g <= 0 scale the state before each token is added. With
// b_t = g_0 + ... + g_t inside a chunk (log2 units here), the prefix state
// reaches query t scaled by 2^{b_t}, key j <= t of the chunk by 2^{b_t - b_j},
// and the state leaves the chunk scaled by 2^{b_last} with key j weighted
// 2^{b_last - b_j}.

constexpr float kLog2e = 1.4426950408889634f;

// 2^x for x <= 0 with v_exp_f32 (results below the fp32 normal range may flush
// to zero, which only drops weights under 2^-126).
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

struct ChunkDecay {
    float b;      // lane t (< C): b_t; lanes past the chunk: b_{C-1}
    float last;   // b_{C-1} (positions past a ragged end carry g = 0)
};

// Inclusive scan of the staged log-decays over the wavefront (lane = position).
template <int C>
__device__ __forceinline__ ChunkDecay chunk_decay(const char* staged_g, const Lane& L) {
    float x = L.lane < C ? reinterpret_cast<const float*>(staged_g)[L.lane] * kLog2e : 0.0f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (L.lane >= d) x += y;
    }
    return ChunkDecay{x, __shfl(x, C - 1, 64)};
}

// The key positions' b values of one chunk, kept in LDS rather than registers
// (one 64-float row per wavefront, rewritten each chunk by the same
// wavefront): b(jb, r) is position 16 jb + 4g + r; last = b_{C-1}.
struct KeyDecay {
    const float* row = nullptr;   // this lane's view of the row: + 4g
    float last = 0.0f;
    __device__ float b(int jb, int r) const { return row[16 * jb + r]; }
};

// Writes the chunk's b (lane = position; lanes past the chunk hold b_{C-1}) to
// this wavefront's row.
__device__ __forceinline__ KeyDecay key_decays(const ChunkDecay& cd, float* wrow, const Lane& L) {
    wrow[L.lane] = cd.b;
    return KeyDecay{wrow + 4 * L.g, cd.last};
}

// Bytes of LDS for the rows of NW wavefronts (gated kernels only).
constexpr int kKeyDecayRowBytes = 64 * 4;

// Chunk c of a segment [c0, c1) lives in buffer (c - c0) % 2 and is staged one
// iteration ahead. Per iteration: a loading wavefront waits for every
// outstanding memory operation of its own (its part of chunk c, and any stores:
// loads and stores may complete out of order, so no partial count is safe),
// then all meet at a barrier (every part has landed and everyone is done with
// the buffer chunk c+1 will overwrite), then chunk c+1 is issued.
template <int DK, int DV, int C, int NW, int NLOAD = NW, bool GATE = false>
struct Pipeline {
    using IO = ChunkIO<DK, DV, C, NW, NLOAD, GATE>;
    char* lds;
    int c0, c1, T;
    size_t tok_base;
    bool with_q;
    const float* gate = nullptr;   // log-decays [.., T] when GATE

    __device__ char* buffer(int c) const { return lds + ((c - c0) & 1) * IO::BUF; }
    __device__ uint32_t buffer_lds(int c) const {
        return lds_address(lds) + ((c - c0) & 1) * IO::BUF;
    }

    __device__ void stage(const bf16_t* q, const bf16_t* k, const bf16_t* v, int c, const Lane& L) {
        if (c >= c1) return;
        const int n = min(C, T - c * C);
        const size_t tok0 = tok_base + (size_t)c * C;
        if (n == C) IO::stage_async(q, k, v, gate, tok0, buffer_lds(c), with_q, L);
        else IO::stage_ragged(q, k, v, gate, tok0, n, buffer(c), with_q, L);
    }
    __device__ void acquire(const bf16_t* q, const bf16_t* k, const bf16_t* v, int c, const Lane& L) {
        if (L.w < NLOAD) wait_vmcnt<0>();
        lds_barrier();
        stage(q, k, v, c + 1, L);
    }

    // Split acquisition for kernels whose loading wavefronts issue no global
    // stores (their loads then complete in issue order, so partial counts are
    // exact): acquire_q makes only the q part of chunk c visible (a loading
    // wavefront lets its k and v copies of chunk c stay in flight), then stages
    // chunk c+1; wait_kv, placed before a later workgroup barrier, waits for
    // the rest of chunk c (everything except the copies of chunk c+1).
    __device__ bool full(int c) const { return c < c1 && T - c * C >= C; }
    __device__ void acquire_q(const bf16_t* q, const bf16_t* k, const bf16_t* v, int c,
                              const Lane& L) {
        if (L.w < NLOAD) wait_vmcnt_upto(full(c) ? IO::kv_pieces(L.w) : 0);
        lds_barrier();
        stage(q, k, v, c + 1, L);
    }
    __device__ void wait_kv(int c, const Lane& L) const {
        if (L.w < NLOAD) wait_vmcnt_upto(full(c + 1) ? IO::issued(L.w, with_q ? 0 : IO::QB / 1024) : 0);
    }
};

// NBUF-deep staging for kernels whose wavefronts issue loads only (k | v of
// chunks, no global stores until the end): chunk c lives in buffer
// (c - c0) % NBUF and is staged NBUF - 1 iterations ahead. Loads of one
// wavefront complete in order, so at chunk c each wavefront waits only until
// no more than its copies of the already-staged later chunks are outstanding,
// then all meet at a barrier and chunk c + NBUF - 1 is issued into the buffer
// chunk c - 1 used.
template <int DK, int DV, int C, int NW, int NBUF, bool GATE = false>
struct LoadPipeline {
    using IO = ChunkIO<DK, DV, C, NW, NW, GATE>;
    static constexpr int PQ = IO::QB / 1024, PV = IO::VB / 1024;
    char* lds;
    int c0, c1, T;
    size_t tok_base;
    const float* gate = nullptr;   // log-decays [.., T] when GATE

    __device__ char* buffer(int c) const { return lds + ((c - c0) % NBUF) * IO::BUF; }
    __device__ uint32_t buffer_lds(int c) const {
        return lds_address(lds) + ((c - c0) % NBUF) * IO::BUF;
    }
    __device__ bool full(int c) const { return c < c1 && T - c * C >= C; }
    // direct-to-LDS copies wavefront w issues for one full chunk (k and v
    // pieces, and the log-decays for wavefront 0 when GATE)
    __device__ static int pieces(int w) { return IO::issued(w, PQ); }
    __device__ void stage(const bf16_t* k, const bf16_t* v, int c, const Lane& L) {
        if (c >= c1) return;
        const int n = min(C, T - c * C);
        const size_t tok0 = tok_base + (size_t)c * C;
        if (n == C) IO::stage_async(nullptr, k, v, gate, tok0, buffer_lds(c), false, L);
        else IO::stage_ragged(nullptr, k, v, gate, tok0, n, buffer(c), false, L);
    }
    __device__ void prologue(const bf16_t* k, const bf16_t* v, const Lane& L) {
#pragma unroll
        for (int i = 0; i < NBUF - 1; ++i) stage(k, v, c0 + i, L);
    }
    __device__ void acquire(const bf16_t* k, const bf16_t* v, int c, const Lane& L) {
        int later = 0;                             // full chunks staged after c
#pragma unroll
        for (int j = 1; j < NBUF - 1; ++j) later += full(c + j) ? 1 : 0;
        wait_vmcnt_upto(later * pieces(L.w));
        lds_barrier();
        stage(k, v, c + NBUF - 1, L);
    }
};

}  // namespace kata
