/*
 * kata.h - C ABI of the MI355X (gfx950) KATA causal-forward library.
 *
 * KATA is normalised kernelised linear attention with the rank-one PSD feature
 * psi(u) = u u^T ("Kernelized Linear Attention: Breaking the Capacity Wall with
 * Symmetric Cones", arXiv 2607.17419; the gist.science explainers, technical
 * summary sections 2.1-2.3, and the paper's abstract). For every batch b, head h
 * and position t:
 *
 *     o_t = sum_{j <= t} (q_t . k_j)^2 v_j  /  sum_{j <= t} (q_t . k_j)^2
 *
 * (j over all positions when causal = 0; o_t = 0 when the denominator is 0).
 * The library computes it in the exact O(T) chunked-state form the explainers
 * describe (section 2.3): a dense masked intra-chunk term, per-chunk states
 * S = phi(K)^T V and z = phi(K)^T 1, and an associative (prefix) scan over chunk
 * states; plus the single-token recurrent step the abstract calls constant-time
 * recurrent inference.
 *
 * Packed feature (state layout). phi(x) has D = d(d+1)/2 entries, in row-major
 * upper-triangle order p(i,j) = i*d - i*(i-1)/2 + (j-i) for i <= j; the entry is
 * x_i*x_j on the diagonal and sqrt(2)*x_i*x_j off it, so phi(q).phi(k) = (q.k)^2.
 * Every state argument (S [.., D, d_v], z [.., D]) uses this layout, in fp32.
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major, last dimension fastest: q, k [B,H,T,d_k],
 *    v, o [B,H,T,d_v]. Element type is `dtype` (fp32 or bf16) for q, k, v, o;
 *    states are always fp32.
 *  - All pointers are device pointers owned by the caller and 16-byte aligned.
 *    The library never allocates device memory: scratch space is the caller's
 *    `workspace`, sized by the matching *_workspace query.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *    the call returns without waiting. Results are valid once the stream has
 *    reached that point.
 *  - Argument errors are reported synchronously and nothing is launched:
 *    KATA_EINVAL (null pointer, misalignment, negative size), KATA_EUNSUPPORTED
 *    (shape outside the supported set), KATA_EWORKSPACE (workspace too small).
 *    A failed launch returns KATA_EHIP.
 *  - Supported shapes: d_k in {16, 32}; d_v in {16, 32, 64}; chunk in
 *    {16, 32, 64, 128}; any T >= 0 (a ragged last chunk covers
 *    [cC, min(cC+C, T))); B, H >= 0. Empty inputs launch nothing except the
 *    state export. Inputs must be finite.
 *  - Inputs and outputs must not overlap, except decode's S and z, which are
 *    updated in place. The library keeps no global state (apart from the static
 *    scratch of kata_chunked_fwd_noalloc) and is thread-safe; calls that share a
 *    workspace must be ordered on one stream.
 */
#ifndef KATA_H
#define KATA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KATA_OK = 0,
    KATA_EINVAL = 1,
    KATA_EUNSUPPORTED = 2,
    KATA_EWORKSPACE = 3,
    KATA_EHIP = 4,
    KATA_ESCRATCH = 5     /* the problem needs more than the static scratch (noalloc call) */
} kata_status_t;

typedef enum { KATA_F32 = 0, KATA_BF16 = 1 } kata_dtype_t;

/* Packed feature dimension D = d(d+1)/2 (the number of unique entries of the
 * symmetric lift x x^T; explainer section 2.2). Returns -1 for d < 0. */
int kata_phi_dim(int d);

/* Human-readable name of a status code (static string). */
const char* kata_status_string(kata_status_t status);

/* Library version string, "major.minor.patch". */
const char* kata_version(void);

/* Bytes of workspace kata_chunked_fwd needs for this problem (0 if none).
 * Returns 0 for unsupported or invalid shapes too; kata_chunked_fwd then
 * reports the precise error. The matrix-core paths cut each (batch, head) into
 * segments of G chunks, about 1024 segments over the whole problem (256 at
 * d_k = 32); kata_chunked_fwd_ex takes G explicitly. */
size_t kata_chunked_fwd_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                  kata_dtype_t dtype, int causal);

/* Chunked causal (or full, causal = 0) forward.
 *   q, k [B,H,T,d_k]; v [B,H,T,d_v] (dtype) - inputs.
 *   o [B,H,T,d_v] (dtype) - output, overwritten.
 *   chunk - the chunk length C of the chunked-state form (section 2.3); the
 *     intra-chunk term covers positions of one chunk, the inter-chunk term the
 *     prefix state of all earlier chunks.
 *   S0 [B,H,D,d_v], z0 [B,H,D] (fp32) - optional initial state standing for
 *     tokens before position 0 (both NULL = zero state; one NULL = KATA_EINVAL).
 *   S_out [B,H,D,d_v], z_out [B,H,D] (fp32) - optional final state S0 + phi(K)^T V
 *     and z0 + phi(K)^T 1 (both NULL = not written; one NULL = KATA_EINVAL).
 *   workspace, ws_bytes - device scratch of at least kata_chunked_fwd_workspace
 *     bytes (may be NULL when that is 0).
 * Output dtype equals input dtype. The mask is inclusive (position t sees j <= t):
 * the explainers' output gate blends the previous readout with the current
 * value (section 2.1).
 * Few keys. Where the inter-chunk prefix may hold only a few keys, its terms
 * phi(q)_p S_p (each up to |q|^2 |k|^2) sum to weights (q.k)^2 that can be far
 * smaller, so the bf16 matrix-core shapes (PSD lift; d_k = 16 with chunk 32 or
 * 64, d_k = 32 with chunk 64 or 128) take those terms with split operands
 * (hi + lo bf16, about 16 significant bits): with an initial state, the first
 * chunk of every head (one extra launch of one chunk per head) and, for a
 * non-causal call within one chunk, every query and the state build. With
 * causal = 0, no initial state and T <= chunk on those shapes, o is evaluated
 * in the quadratic form (as kata_flash_fwd), every (q.k)^2 in fp32; the final
 * state is formed as otherwise. */
kata_status_t kata_chunked_fwd(const void* q, const void* k, const void* v, void* o,
                               int B, int H, int T, int d_k, int d_v, int chunk, int causal,
                               kata_dtype_t dtype,
                               const float* S0, const float* z0,
                               float* S_out, float* z_out,
                               void* workspace, size_t ws_bytes, void* stream);

/* kata_chunked_fwd with phase timing: identical work and results, and it also
 * records events[0..4] (hipEvent_t, created by the caller) on `stream` at the
 * phase boundaries - events[0] before the chunk-state phase, events[1] after it,
 * events[2] after the inter-chunk scan, events[3] after the output kernel,
 * events[4] after the final-state export (S_out, z_out; an empty phase when they
 * are NULL) - so a caller can time each phase with hipEventElapsedTime.
 * n_events must be >= 5 (else KATA_EINVAL); events after the fifth are ignored. */
kata_status_t kata_chunked_fwd_profiled(const void* q, const void* k, const void* v, void* o,
                                        int B, int H, int T, int d_k, int d_v, int chunk,
                                        int causal, kata_dtype_t dtype,
                                        const float* S0, const float* z0,
                                        float* S_out, float* z_out,
                                        void* workspace, size_t ws_bytes, void* stream,
                                        void* const* events, int n_events);

/* Feature map of kata_chunked_fwd_ex.
 *  KATA_FEATURE_PSD: the rank-one PSD lift above (weights (q.k)^2; state
 *    dimension D = d(d+1)/2, packed) - what kata_chunked_fwd computes.
 *  KATA_FEATURE_IDENTITY: the first-order feature phi1(x) = x, the baseline the
 *    paper's abstract sets the PSD lift's scan against (weights q.k; state
 *    dimension d_k, S [.., d_k, d_v] row-major and z [.., d_k]). The output keeps
 *    the normalised form o_t = sum_j (q_t.k_j) v_j / sum_j (q_t.k_j), 0 where the
 *    denominator is 0; it is a convex combination when the weights are
 *    nonnegative (queries and keys in the nonnegative orthant, the cone of this
 *    feature in explainer section 2.2). */
typedef enum { KATA_FEATURE_PSD = 0, KATA_FEATURE_IDENTITY = 1 } kata_feature_t;

/* How the inter-chunk prefix is formed (explainer section 2.3: recurrence depth
 * O(N_C) sequentially, O(log N_C) with an associative scan).
 *  KATA_PREFIX_SCAN: chunk states of parallel segments, an associative scan over
 *    them, then every segment's output in parallel (kata_chunked_fwd). The scan
 *    over segment states is blocked (records summed in runs of 16, groups of 8
 *    runs, tiles of 128 records chained), the fastest at the segment counts the
 *    library plans (about 1024 segments); its depth grows with the number of
 *    tiles.
 *  KATA_PREFIX_SEQUENTIAL: one workgroup per (batch, head) walks every chunk in
 *    order, carrying the state from chunk to chunk (depth N_C). Same results up
 *    to fp32 summation order. bf16 only.
 *  KATA_PREFIX_TREE: as KATA_PREFIX_SCAN with a log-depth scan over segment (or,
 *    on the fp32 path, chunk) states: a Kogge-Stone scan within tiles of 128
 *    states, reduce-then-scan across tiles (ceil(log2 n) combine levels per tile
 *    pass and one per level of tiles; kata_prefix_depth reports it). */
typedef enum { KATA_PREFIX_SCAN = 0, KATA_PREFIX_SEQUENTIAL = 1, KATA_PREFIX_TREE = 2 } kata_prefix_t;

/* Depth of the inter-chunk prefix of a kata_chunked_fwd_ex call with these
 * arguments: the number of dependent state combines on its longest chain - the
 * chunks a segment's workgroup carries in order plus the levels of the scan
 * over segment states (matrix-core paths), the scan levels over chunk states
 * (fp32 path), or every chunk (KATA_PREFIX_SEQUENTIAL). -1 for invalid or
 * unsupported arguments. */
int kata_prefix_depth(int B, int H, int T, int d_k, int d_v, int chunk, kata_dtype_t dtype,
                      kata_feature_t feature, kata_prefix_t prefix, int segment_chunks);

/* State dimension of a feature: d(d+1)/2 for KATA_FEATURE_PSD, d for
 * KATA_FEATURE_IDENTITY; -1 for d < 0 or an unknown feature. */
int kata_feature_dim(int d, kata_feature_t feature);

/* Workspace of kata_chunked_fwd_ex (0 if none or if the arguments are invalid);
 * segment_chunks as there (it sets the number of segment records). */
size_t kata_chunked_fwd_ex_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                     kata_dtype_t dtype, int causal, kata_feature_t feature,
                                     kata_prefix_t prefix, int segment_chunks);

/* kata_chunked_fwd with a choice of feature map and prefix method; every other
 * argument as there, with the state dimension of `feature` in S0, z0, S_out,
 * z_out. KATA_FEATURE_PSD with KATA_PREFIX_SCAN and segment_chunks = 0 is
 * kata_chunked_fwd.
 * segment_chunks - G, the chunks per segment of the matrix-core scan paths
 *   (each segment's state is built by one workgroup and the associative scan
 *   runs over segment states); 0 = automatic (about one resident wave of
 *   workgroups), negative = KATA_EINVAL. The same value must be given to the
 *   workspace query. Ignored by the sequential prefix and the fp32 path.
 * KATA_PREFIX_SEQUENTIAL needs a shape of a bf16 matrix-core path (else
 * KATA_EUNSUPPORTED): for KATA_FEATURE_PSD d_k = 16 with chunk 32 or 64, d_k = 32
 * with chunk 64 or 128; for KATA_FEATURE_IDENTITY chunk 32, 64 or 128. Every
 * other supported shape (fp32 inputs, or chunk 16 with the identity feature)
 * runs the fp32 path with KATA_PREFIX_SCAN or KATA_PREFIX_TREE (over one state
 * per chunk). */
kata_status_t kata_chunked_fwd_ex(const void* q, const void* k, const void* v, void* o,
                                  int B, int H, int T, int d_k, int d_v, int chunk, int causal,
                                  kata_dtype_t dtype, kata_feature_t feature,
                                  kata_prefix_t prefix, int segment_chunks,
                                  const float* S0, const float* z0,
                                  float* S_out, float* z_out,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Decay-gated chunked forward (causal). The pages name decay gates among the
 * mechanisms whose interaction with the feature geometry the paper studies (the
 * abstract) and describe gated linear RNNs with learned forget gates (explainer
 * section 1), but print no formula; the reading implemented is a scalar forget
 * gate per token and head that scales the whole state before the token is added:
 *     S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T,  z_t = exp(g_t) z_{t-1} + phi(k_t),
 *     o_t = phi(q_t).S_t / phi(q_t).z_t   (0 where the denominator is 0),
 * i.e. weights (q_t.k_j)^2 exp(g_{j+1} + ... + g_t), still nonnegative.
 *   log_decay [B,H,T] (fp32, device) - g, every value <= 0 (finite, or very
 *     negative for a reset).
 *   prefix - KATA_PREFIX_SCAN (segment states, then an associative scan under
 *     the non-commutative operator (a1,S1) o (a2,S2) = (a1 a2, a2 S1 + S2)) or
 *     KATA_PREFIX_SEQUENTIAL (one workgroup per head walks every chunk).
 * Every other argument as for kata_chunked_fwd (S0, z0 stand for earlier tokens
 * and decay with the sequence; S_out, z_out are the decayed final state).
 * Paths: dtype KATA_BF16 with d_k = 16 and chunk in {32, 64}, or d_k = 32 and
 * chunk in {64, 128}, runs on the matrix cores with any prefix method (the
 * tree scan combines segment states under the same operator), provided T
 * is a multiple of 4 or B*H == 1 (the log-decays of a head are copied 16 bytes
 * at a time). Every other supported shape (d_k in {16, 32}, d_v in {16, 32, 64},
 * chunk in {16, 32, 64, 128}, fp32 or bf16 inputs, any T) runs the fp32 path
 * (fp32 arithmetic throughout), with KATA_PREFIX_SCAN only. Else KATA_EUNSUPPORTED. */
size_t kata_chunked_fwd_decay_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                        kata_dtype_t dtype, kata_prefix_t prefix);
kata_status_t kata_chunked_fwd_decay(const void* q, const void* k, const void* v,
                                     const float* log_decay, void* o,
                                     int B, int H, int T, int d_k, int d_v, int chunk,
                                     kata_dtype_t dtype, kata_prefix_t prefix,
                                     const float* S0, const float* z0,
                                     float* S_out, float* z_out,
                                     void* workspace, size_t ws_bytes, void* stream);

/* kata_chunked_fwd_decay with a choice of feature map and segment length:
 * KATA_FEATURE_PSD with segment_chunks = 0 is kata_chunked_fwd_decay;
 * KATA_FEATURE_IDENTITY gates the first-order feature phi1(x) = x (weights
 * (q_t.k_j) exp(g_{j+1} + ... + g_t), state d_k x d_v in S0, z0, S_out, z_out):
 * on the matrix cores for dtype KATA_BF16 with chunk 32 or 64 (either prefix;
 * T a multiple of 4 or B*H == 1), else on the fp32 path with KATA_PREFIX_SCAN.
 * segment_chunks as for kata_chunked_fwd_ex. Every other argument, error and
 * layout as kata_chunked_fwd_decay. The gated PSD matrix-core kernels take
 * split (hi + lo bf16) operands for every lifted query, key, state entry and
 * Gram product: strong gates leave only a few keys in the state. */
size_t kata_chunked_fwd_decay_ex_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                           kata_dtype_t dtype, kata_feature_t feature,
                                           kata_prefix_t prefix, int segment_chunks);
kata_status_t kata_chunked_fwd_decay_ex(const void* q, const void* k, const void* v,
                                        const float* log_decay, void* o, int B, int H, int T,
                                        int d_k, int d_v, int chunk, kata_dtype_t dtype,
                                        kata_feature_t feature, kata_prefix_t prefix,
                                        int segment_chunks,
                                        const float* S0, const float* z0, float* S_out,
                                        float* z_out, void* workspace, size_t ws_bytes,
                                        void* stream);

/* kata_decode_step with the decay gate above: log_decay [N] (fp32, device), and
 * S = exp(g) S + phi(k) v^T, z = exp(g) z + phi(k) before the read. Same shapes,
 * dtypes and errors as kata_decode_step (log_decay NULL = KATA_EINVAL). */
kata_status_t kata_decode_step_decay(const void* q, const void* k, const void* v,
                                     const float* log_decay, float* S, float* z, void* o,
                                     int N, int d_k, int d_v, kata_dtype_t dtype, void* stream);

/* Bytes of workspace kata_scan_states needs (0 for the fp32 path). */
size_t kata_scan_states_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                  kata_dtype_t dtype);

/* Per-chunk states and their exclusive prefix (the associative scan over chunk
 * states, section 2.3; operator +, identity S0 or 0). bf16 inputs on the
 * matrix-core shapes (d_k = 16 with chunk 32 or 64, d_k = 32 with chunk 64 or
 * 128) take segment states, an associative scan over them and a walk of each
 * segment that writes every chunk's prefix, with split (hi + lo) operands for
 * the lifted keys, so the prefixes are exact sums up to fp32 rounding; every
 * other shape the fp32 path (per-chunk states, then the scan over them).
 *   workspace, ws_bytes - at least kata_scan_states_workspace bytes.
 *   k [B,H,T,d_k], v [B,H,T,d_v] (dtype) - inputs.
 *   S_prefix [B,H,NC,D,d_v], z_prefix [B,H,NC,D] (fp32, NC = ceil(T/chunk)) -
 *     output: entry c holds S0 + sum over chunks c' < c of phi(K_c')^T V_c'
 *     (likewise z). Both required when NC > 0.
 *   S0, z0 - optional initial state (as kata_chunked_fwd).
 *   S_out, z_out - optional total state after the last chunk. */
kata_status_t kata_scan_states(const void* k, const void* v,
                               int B, int H, int T, int d_k, int d_v, int chunk,
                               kata_dtype_t dtype,
                               const float* S0, const float* z0,
                               float* S_prefix, float* z_prefix,
                               float* S_out, float* z_out,
                               void* workspace, size_t ws_bytes, void* stream);

/* Quadratic ("flash-style") forward: the same o as kata_chunked_fwd, evaluated
 * directly as sum_{j <= t} (q_t.k_j)^2 v_j / sum_{j <= t} (q_t.k_j)^2 by
 * streaming key blocks past tiles of queries (the quadratic KATA forward
 * of the explainers, section 4, and the abstract), with no chunk states. It
 * takes no initial state and keeps no final state.
 *   q, k [B,H,T,d_k]; v, o [B,H,T,d_v] - bf16 only (fp32 inputs return
 *     KATA_EUNSUPPORTED); d_k in {16, 32}, d_v in {16, 32, 64}.
 *   causal - as kata_chunked_fwd (inclusive mask when nonzero).
 * Work grows as T^2 / 2 per (b, h); no workspace. */
kata_status_t kata_flash_fwd(const void* q, const void* k, const void* v, void* o,
                             int B, int H, int T, int d_k, int d_v, int causal,
                             kata_dtype_t dtype, void* stream);

/* One recurrent decode step for N independent (sequence, head) rows: the
 * constant-time recurrent inference of the abstract, with a fixed-size state.
 *   q, k [N,d_k]; v [N,d_v] (dtype) - the new token.
 *   S [N,D,d_v], z [N,D] (fp32) - state, updated in place:
 *     S += phi(k) v^T, z += phi(k).
 *   o [N,d_v] (dtype) - output phi(q).S / phi(q).z, read after the update
 *     (the token attends to itself), 0 when the denominator is 0. */
kata_status_t kata_decode_step(const void* q, const void* k, const void* v,
                               float* S, float* z, void* o,
                               int N, int d_k, int d_v, kata_dtype_t dtype, void* stream);

/* DeltaKATA forward (causal): the delta-rule variant the explainers name for
 * repeated-key overwrite (section 4; no formula is printed). Reading built:
 * with the unit-norm lifted key kappa_t = phi(k_t) / |k_t|^2 (0 for k = 0) and
 * a write strength beta_t, the numerator and denominator states form one
 * augmented state A = [S | z] updated by the delta rule of DeltaNet with the
 * value [v_t, 1]:
 *     A_t = A_{t-1} + beta_t kappa_t ([v_t, 1] - kappa_t^T A_{t-1}),
 *     o_t = phi(q_t).S_t / phi(q_t).z_t     (0 where the denominator is 0).
 * beta = 1 makes the state return exactly v_t for the key k_t; mutually
 * orthogonal unit keys with beta = 1 give kata_chunked_fwd's output. The
 * erase can make weights negative, so outputs need not be convex combinations.
 *   q, k [B,H,T,d_k]; v, o [B,H,T,d_v] (dtype) - as kata_chunked_fwd.
 *   beta [B,H,T] (fp32, device) - write strengths, expected in [0, 1].
 *   chunk - 16, 32 or 64: chunks are walked in order (the state transition is
 *     matrix-affine); inside a chunk a unit lower-triangular system gives the
 *     tokens' writes. Its inverse depends only on the chunk's keys and write
 *     strengths, so a first kernel forms it for every chunk at once (blocks of
 *     16, by forward substitution); the walk then does four matrix products
 *     per chunk.
 *   S0, z0 / S_out, z_out - optional initial / final state as kata_chunked_fwd
 *     (the packed layout; both of a pair or neither).
 *   workspace - device memory of kata_delta_fwd_workspace() bytes, 16-byte
 *     aligned, owned by the caller (NULL only when B*H*T == 0); it holds each
 *     chunk's inverse and masked weights between the two kernels.
 * d_k in {16, 32}, d_v in {16, 32, 64}, fp32 or bf16 inputs, any T >= 0; fp32
 * arithmetic throughout. The walk runs one workgroup per (batch, head, 15 value
 * columns plus the denominator column). Errors as kata_chunked_fwd (chunk 128:
 * KATA_EUNSUPPORTED; a short workspace: KATA_EWORKSPACE). */
kata_status_t kata_delta_fwd(const void* q, const void* k, const void* v, const float* beta,
                             void* o, int B, int H, int T, int d_k, int d_v, int chunk,
                             kata_dtype_t dtype, const float* S0, const float* z0,
                             float* S_out, float* z_out, void* workspace, size_t ws_bytes,
                             void* stream);

/* Bytes of workspace kata_delta_fwd needs for this shape: 8 C^2 per (batch,
 * head, chunk); 0 for an unsupported shape. */
size_t kata_delta_fwd_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                kata_dtype_t dtype);

/* One DeltaKATA decode step for N rows: [S | z] += beta kappa ([v, 1] -
 * kappa^T [S | z]) in place, then o = phi(q).S / phi(q).z. Shapes, dtypes and
 * errors as kata_decode_step; beta [N] (fp32, device; NULL = KATA_EINVAL). */
kata_status_t kata_decode_step_delta(const void* q, const void* k, const void* v,
                                     const float* beta, float* S, float* z, void* o, int N,
                                     int d_k, int d_v, kata_dtype_t dtype, void* stream);

/* Factored PSD features, KATA-Mg and KATA-Sigma-g: the variants the
 * explainers name (technical summary 2.3, "Variants": multiple PSD factors and
 * summed PSD factors, trading state size against packing efficiency) without
 * printing a construction. Reading built: q and k (width d_k) are cut into g
 * contiguous factors x_a = x[a p, (a+1) p), p = d_k / g, each lifted to the
 * rank-one PSD matrix x_a x_a^T of section 2.2.
 *   KATA_FACTORS_MULTI (KATA-Mg): the factors stay apart, feature
 *     diag(x_1 x_1^T, ..., x_g x_g^T), weight sum_a (q_a . k_a)^2; packed as the
 *     g packed lifts of the factors one after the other (D = g p(p+1)/2).
 *   KATA_FACTORS_SUMMED (KATA-Sigma-g): the factors summed into one p x p
 *     matrix sum_a x_a x_a^T, weight sum_{a,b} (q_a . k_b)^2; packed like one
 *     lift of width p (D = p(p+1)/2).
 * Each factor's lift uses the packing above (row-major upper triangle, sqrt(2)
 * off the diagonal). Both weights are sums of squares, and g = 1 is plain KATA
 * for both. The output is the normalised form of kata_chunked_fwd with these
 * weights. */
typedef enum { KATA_FACTORS_MULTI = 0, KATA_FACTORS_SUMMED = 1 } kata_factors_t;

/* Feature dimension D of a factored feature; -1 when d < 0, g < 1, g does not
 * divide d, or the kind is unknown. */
int kata_factored_dim(int d, int g, kata_factors_t kind);

/* Bytes of workspace kata_factored_fwd needs (0 if none, or for an invalid or
 * unsupported problem). */
size_t kata_factored_fwd_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                   kata_dtype_t dtype, int causal, int g, kata_factors_t kind);

/* Chunked forward (causal, or full with causal = 0) with a factored feature.
 * Arguments, layouts and errors as kata_chunked_fwd; S0, z0, S_out, z_out are
 * [B,H,D,d_v] / [B,H,D] in the factored packed layout (D = kata_factored_dim).
 * g = 1 is kata_chunked_fwd itself (same workspace). For g > 1 the matrix-core
 * path serves bf16 inputs, chunk 64, d_v 32 or 64, and (d_k, g) in {(16, 2),
 * (16, 4), (32, 4)} for both kinds and (32, 2) summed (D <= 144); other shapes
 * return KATA_EUNSUPPORTED, g not dividing d_k KATA_EINVAL. Intra-chunk
 * weights are formed from the factors' inner products in fp32; the lifted
 * features and the state enter the matrix cores as split bf16 operands
 * (hi + lo), so few keys in the prefix cost no accuracy. */
kata_status_t kata_factored_fwd(const void* q, const void* k, const void* v, void* o,
                                int B, int H, int T, int d_k, int d_v, int chunk, int causal,
                                kata_dtype_t dtype, int g, kata_factors_t kind,
                                const float* S0, const float* z0, float* S_out, float* z_out,
                                void* workspace, size_t ws_bytes, void* stream);

/* One recurrent decode step with a factored feature, as kata_decode_step:
 * S [N,D,d_v], z [N,D] updated in place (S += phi(k) v^T, z += phi(k)), then
 * o = phi(q).S / phi(q).z. fp32 or bf16 inputs; d_v in {16, 32, 64}; (d_k, g)
 * as kata_factored_fwd; g = 1 is kata_decode_step. */
kata_status_t kata_decode_step_factored(const void* q, const void* k, const void* v,
                                        float* S, float* z, void* o, int N, int d_k, int d_v,
                                        int g, kata_factors_t kind, kata_dtype_t dtype,
                                        void* stream);

/* Bytes of the library's static device scratch (per GPU) used by
 * kata_chunked_fwd_noalloc. */
#define KATA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* kata_chunked_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as kata_chunked_fwd, without the
 * workspace: the scratch (segment records, initial and final state records)
 * lives in a static device array of KATA_NOALLOC_SCRATCH_BYTES that each GPU
 * the library runs on holds until the process ends (its address is looked up
 * once per device, on the first call made with that device current). The
 * call allocates nothing and calls no allocating routine.
 *   Problems whose kata_chunked_fwd_workspace exceeds
 *   KATA_NOALLOC_SCRATCH_BYTES return KATA_ESCRATCH, with nothing launched
 *   (e.g. B1 H8 T131072 d_k16 d_v64 C64 needs 39.4 MB and fits).
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents (nothing in it has to start at zero). Calls that overlap on one
 *   GPU - on different streams, or from threads without ordering - race;
 *   order them on one stream. A failed device-symbol lookup returns KATA_EHIP. */
kata_status_t kata_chunked_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                       int B, int H, int T, int d_k, int d_v, int chunk,
                                       int causal, kata_dtype_t dtype,
                                       const float* S0, const float* z0,
                                       float* S_out, float* z_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KATA_H */
