// Host-side launchers of the KATA kernels. Each returns hipSuccess or the
// launch error; argument checking happens in kata_api.cpp before any call.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kata {

struct Shape {
    int B, H, T, dk, dv, C;
    int D;    // dk * (dk + 1) / 2
    int NC;   // ceil(T / C)
    bool bf16;
};

// ---- fp32 path (any supported shape; fp32 or bf16 inputs, fp32 math) ----

// Per-chunk totals phi(K_c)^T V_c and phi(K_c)^T 1 in packed layout:
// S_rec [BH, NC, D, dv], z_rec [BH, NC, D]. gdec: per-token log-decays
// [BH, T] or NULL; with them each token is weighted by its decay to the chunk
// end and cdec [BH, NC] receives each chunk's total decay factor. ident: the
// identity feature (D = d_k, s.D must say so) instead of the PSD lift.
hipError_t launch_chunk_states_valu(const Shape& s, const void* k, const void* v,
                                    const float* gdec, float* S_rec, float* z_rec, float* cdec,
                                    int ident, hipStream_t st);

// Chunked forward reading per-chunk exclusive prefixes (causal) or one total
// state per head (non-causal: S_rec [BH, D, dv], z_rec [BH, D]). gdec as above
// (causal only); ident as above.
hipError_t launch_fwd_valu(const Shape& s, const void* q, const void* k, const void* v,
                           const float* gdec, const float* S_rec, const float* z_rec, void* o,
                           int causal, int ident, hipStream_t st);

// ---- associative scan over records (layout-agnostic, fp32) ----

// For each of `nseq` independent sequences of NR records of E floats (record r
// of sequence b at rec + (b*NR + r)*E): replaces every record by the exclusive
// prefix sum init_b + sum_{r' < r} rec_{r'} (init = 0 when NULL; init_b at
// init + b*E). Writes the inclusive total of every sequence to total_a and/or
// total_b (each NULL or E floats per sequence).
// ex (optional): also writes each sequence's total, converted from the record
// layout `ex->layout` to the packed state ex->S [nseq, D, dv], ex->z [nseq, D].
struct RecordExport;
hipError_t launch_scan_records(float* rec, int nseq, int NR, int E, const float* init,
                               float* total_a, float* total_b, hipStream_t st,
                               const RecordExport* ex = nullptr);

// The same with the decay gate: record r of sequence b also carries the factor
// dec[b*NR + r] by which its span decays the state before it; record r becomes
// the exclusive prefix under (a1, S1) o (a2, S2) = (a1 a2, a2 S1 + S2).
hipError_t launch_scan_records_decay(float* rec, const float* dec, int nseq, int NR, int E,
                                     const float* init, float* total_a, float* total_b,
                                     hipStream_t st, const RecordExport* ex = nullptr);

// Log-depth variant of both (dec NULL = plain addition): a Kogge-Stone scan
// within tiles of 128 records, reduce-then-scan across tiles. scratch: at least
// scan_tree_scratch_floats floats (none for NR <= 128). Its depth is checked
// against ceil(log2 NR) plus two combines per level of tiles.
hipError_t launch_scan_records_tree(float* rec, const float* dec, int nseq, int NR, int E,
                                    const float* init, float* total_a, float* total_b,
                                    float* scratch, hipStream_t st,
                                    const RecordExport* ex = nullptr);
size_t scan_tree_scratch_floats(int nseq, int NR, int E, bool decay);
// Dependent combine levels over NR records: method 0 the blocked scan, 1 the
// sequential walk, 2 the tree.
int scan_levels(int NR, int method);

// Record layouts of the matrix-core kernels (kata_records.h) and a packed
// state to export a record to.
constexpr int kRecNone = 0, kRecPsd16 = 1, kRecPsd32 = 2, kRecIdent = 3;
struct RecordExport {
    int layout;      // kRecPsd16, kRecPsd32 or kRecIdent
    int dk, dv;      // kRecIdent: dk = the feature count (rows) of the record
    float* S;        // [nseq, D, dv]
    float* z;        // [nseq, D]
};

// Copies (src != NULL) or zero-fills n floats.
hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st);

// ---- bf16 matrix-core path, d_k = 16 (two wavefronts per segment of G chunks) ----

bool mfma16_supported(const Shape& s);
// floats per state record (accumulator order, see kata_fwd16.hip)
int mfma16_record_floats(int dv);
// rec [BH, NSEG, REC]: total state of every segment. prec: split (hi + lo)
// operands for the lifted keys (exact for bf16 keys), so the records are
// fp32-accurate sums.
hipError_t launch_seg_state16(const Shape& s, const void* k, const void* v, float* rec, int G,
                              int NSEG, bool prec, hipStream_t st);
// causal: prefix [BH, NSEG, REC] exclusive segment prefixes; else prefix [BH, REC] totals
// final_rec (NULL or [BH, REC]): causal only, the running state after each
// head's last segment (the final state when NSEG == 1)
// prec: split (hi + lo) bf16 operands for the inter-chunk term phi(Q).S, the
// Gram denominator and the state update (about three times their matrix work).
// With G = 1 and a grid of one segment per head it recomputes only the first
// chunk of every head from `prefix` (the initial-state record).
hipError_t launch_fwd16(const Shape& s, const void* q, const void* k, const void* v,
                        const float* prefix, float* final_rec, void* o, int causal, int G,
                        int NSEG, bool prec, hipStream_t st);
// Decay-gated (causal only): gdec [BH, T] per-token log-decays (<= 0); the state
// kernel also writes each segment's total decay to segdec [BH, NSEG]. The gated
// kernels always take split operands (a strong gate leaves a few keys in the
// state, whose bf16 rounding would not average out).
hipError_t launch_seg_state16_decay(const Shape& s, const void* k, const void* v,
                                    const float* gdec, float* rec, float* segdec, int G, int NSEG,
                                    hipStream_t st);
hipError_t launch_fwd16_decay(const Shape& s, const void* q, const void* k, const void* v,
                              const float* gdec, const float* prefix, float* final_rec, void* o,
                              int G, int NSEG, hipStream_t st);
// Per-chunk exclusive prefixes for kata_scan_states: prefix [BH, NSEG, REC]
// scanned (exclusive) segment records; writes the packed prefix of every chunk
// to Sp [BH, NC, D, dv], zp [BH, NC, D] (split key operands: fp32-accurate).
hipError_t launch_prefix16(const Shape& s, const void* k, const void* v, const float* prefix,
                           float* Sp, float* zp, int G, int NSEG, hipStream_t st);
hipError_t launch_record_from_packed16(float* rec, const float* S, const float* z, int dv,
                                       int nrec, hipStream_t st);
hipError_t launch_record_to_packed16(const float* rec, float* S, float* z, int dv, int nrec,
                                     hipStream_t st);

// ---- bf16 matrix-core path, d_k = 32 (four wavefronts per segment of G chunks) ----

bool mfma32_supported(const Shape& s);
int mfma32_record_floats(int dv);
// prec as for d_k = 16
hipError_t launch_seg_state32(const Shape& s, const void* k, const void* v, float* rec, int G,
                              int NSEG, bool prec, hipStream_t st);
// final_rec (NULL or [BH, REC]): causal only, the running state after each
// head's last segment (the final state when NSEG == 1). prec as for d_k = 16
// (the split state is published in two passes of half the tiles each).
hipError_t launch_fwd32(const Shape& s, const void* q, const void* k, const void* v,
                        const float* prefix, float* final_rec, void* o, int causal, int G,
                        int NSEG, bool prec, hipStream_t st);
// Decay-gated (causal only, as for d_k = 16, split operands): gdec [BH, T]
// per-token log-decays (<= 0); the state kernel also writes each segment's
// total decay to segdec [BH, NSEG].
hipError_t launch_seg_state32_decay(const Shape& s, const void* k, const void* v,
                                    const float* gdec, float* rec, float* segdec, int G, int NSEG,
                                    hipStream_t st);
hipError_t launch_fwd32_decay(const Shape& s, const void* q, const void* k, const void* v,
                              const float* gdec, const float* prefix, float* final_rec, void* o,
                              int G, int NSEG, hipStream_t st);
hipError_t launch_prefix32(const Shape& s, const void* k, const void* v, const float* prefix,
                           float* Sp, float* zp, int G, int NSEG, hipStream_t st);
hipError_t launch_record_from_packed32(float* rec, const float* S, const float* z, int dv,
                                       int nrec, hipStream_t st);
hipError_t launch_record_to_packed32(const float* rec, float* S, float* z, int dv, int nrec,
                                     hipStream_t st);

// ---- bf16 matrix-core path, first-order (identity) feature ----
bool first_supported(const Shape& s);
int first_record_floats(int dk, int dv);
hipError_t launch_seg_state1(const Shape& s, const void* k, const void* v, float* rec, int G,
                             int NSEG, hipStream_t st);
// split (causal only): one workgroup per (segment, head, 16-column value tile),
// each evaluating its tile's columns (and the denominator); used by the
// sequential walk, whose one segment per head leaves compute units idle.
hipError_t launch_fwd1(const Shape& s, const void* q, const void* k, const void* v,
                       const float* prefix, float* final_rec, void* o, int causal, int G,
                       int NSEG, hipStream_t st, bool split = false);
// Decay-gated variants (causal, chunk 32 or 64): gdec [BH, T] log-decays;
// the state kernel also writes each segment's decay factor to segdec [BH, NSEG].
bool first_decay_supported(const Shape& s);
hipError_t launch_seg_state1_decay(const Shape& s, const void* k, const void* v, const float* gdec,
                                   float* rec, float* segdec, int G, int NSEG, hipStream_t st);
hipError_t launch_fwd1_decay(const Shape& s, const void* q, const void* k, const void* v,
                             const float* gdec, const float* prefix, float* final_rec, void* o,
                             int G, int NSEG, hipStream_t st, bool split = false);
hipError_t launch_record_from_packed1(float* rec, const float* S, const float* z, int dk, int dv,
                                      int nrec, hipStream_t st);
hipError_t launch_record_to_packed1(const float* rec, float* S, float* z, int dk, int dv, int nrec,
                                    hipStream_t st);

// ---- quadratic (flash-style) forward, bf16 ----
bool flash_supported(const Shape& s);
hipError_t launch_flash_fwd(const Shape& s, const void* q, const void* k, const void* v, void* o,
                            int causal, hipStream_t st);

// ---- DeltaKATA (delta rule on [S | z], fp32 arithmetic) ----
bool delta_supported(const Shape& s);
// Workspace of the forward: each chunk's diag(Inv) T and masked weights,
// 2 C^2 floats per (batch*head, chunk).
size_t delta_workspace_bytes(const Shape& s);
// beta [BH, T]; S0, z0 / S_out, z_out packed states or NULL; ws of
// delta_workspace_bytes(s), 16-byte aligned
hipError_t launch_delta_fwd(const Shape& s, const void* q, const void* k, const void* v,
                            const float* beta, void* o, const float* S0, const float* z0,
                            float* S_out, float* z_out, float* ws, hipStream_t st);
hipError_t launch_delta_decode(const void* q, const void* k, const void* v, const float* beta,
                               float* S, float* z, void* o, int N, int dk, int dv, bool bf16,
                               hipStream_t st);

// ---- factored PSD features (KATA-Mg: summed = false, KATA-Sigma-g: summed = true) ----
// G factors of width d_k / G; bf16, chunk 64, d_v 32 or 64; feature dimension
// at most 144 (d_k 16 with G 2 or 4, d_k 32 with G 4, d_k 32 with G 2 summed).
int factored_dim(int dk, int G, bool summed);
bool factored_supported(const Shape& s, int G, bool summed);
bool factored_decode_supported(int dk, int dv, int G, bool summed);
// floats per record: feature tiles x (value tiles + z tile) x 256, layout of
// the first-order records (kRecIdent export with dk = the feature dimension)
int factored_record_floats(int dk, int dv, int G, bool summed);
hipError_t launch_fact_seg_state(const Shape& s, int G, bool summed, const void* k, const void* v,
                                 float* rec, int Gs, int NSEG, hipStream_t st);
hipError_t launch_fact_fwd(const Shape& s, int G, bool summed, const void* q, const void* k,
                           const void* v, const float* prefix, void* o, int causal, int Gs,
                           int NSEG, hipStream_t st);
hipError_t launch_fact_record_from_packed(float* rec, const float* S, const float* z, int D,
                                          int dv, int REC, int nrec, hipStream_t st);
hipError_t launch_fact_record_to_packed(const float* rec, float* S, float* z, int D, int dv,
                                        int REC, int nrec, hipStream_t st);
hipError_t launch_fact_decode(const void* q, const void* k, const void* v, float* S, float* z,
                              void* o, int N, int dk, int dv, int G, bool summed, bool bf16,
                              hipStream_t st);

// ---- decode ----
// g: NULL, or [N] per-row log-decays (S = exp(g) S + phi(k) v^T, z likewise)
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g, float* S,
                         float* z, void* o, int N, int dk, int dv, bool bf16, hipStream_t st);

}  // namespace kata
