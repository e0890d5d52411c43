// C ABI of the KATA library: argument checking, workspace planning and launch
// orchestration. Every kernel runs on the caller's stream; nothing here
// allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/kata.h"
#include "kata_internal.h"

namespace {

using kata::Shape;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dk(int d) { return d == 16 || d == 32; }
bool supported_dv(int d) { return d == 16 || d == 32 || d == 64; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Checks sizes and the shape set; fills s (s->D is the state dimension of the
// feature: d(d+1)/2 for the PSD lift, d for the identity).
kata_status_t make_shape(int B, int H, int T, int dk, int dv, int C, kata_dtype_t dt, Shape* s,
                         kata_feature_t f = KATA_FEATURE_PSD) {
    if (B < 0 || H < 0 || T < 0 || dk < 0 || dv < 0 || C <= 0) return KATA_EINVAL;
    if (dt != KATA_F32 && dt != KATA_BF16) return KATA_EINVAL;
    if (!supported_dk(dk) || !supported_dv(dv) || !supported_chunk(C)) return KATA_EUNSUPPORTED;
    // indices are 64-bit in the kernels; keep grid dimensions in range
    if ((int64_t)B * H > 65535 || T > (1 << 28)) return KATA_EUNSUPPORTED;
    s->B = B; s->H = H; s->T = T; s->dk = dk; s->dv = dv; s->C = C;
    s->D = f == KATA_FEATURE_IDENTITY ? dk : dk * (dk + 1) / 2;
    s->NC = (T + C - 1) / C;
    s->bf16 = dt == KATA_BF16;
    return KATA_OK;
}

// Launch plan of kata_chunked_fwd(_ex) and its workspace layout.
//  VALU path (fp32 inputs, shapes without a matrix-core kernel; PSD lift with
//    the scan only): per-chunk records in packed layout, scanned over chunks.
//  Matrix-core paths (bf16; PSD lift with d_k = 16 or 32, or the identity
//    feature): per-segment records of G chunks in accumulator order, an
//    initial-state record and a total record per head. The sequential prefix
//    is one segment of every chunk per head.
struct FwdPlan {
    bool ok;    // supported combination of shape, feature and prefix method
    int mfma;   // 0 (VALU path), 16 or 32 (PSD lift, d_k), 1 (identity feature)
    bool seq;   // sequential prefix
    bool tree;  // log-depth scan
    int G, NSEG, REC;
    size_t S_off, z_off, init_off, total_off, tree_off, bytes;
};

// G for a requested value (> 0) or automatically (0): about `workgroups`
// segments in flight (one wave of resident workgroups over the 256 compute
// units), each on a run of chunks.
int segment_chunks(const Shape& s, int workgroups, int requested) {
    if (requested > 0) return requested;
    const long long chunks = (long long)s.B * s.H * s.NC;
    return (int)std::max<long long>(1, chunks / workgroups);
}

FwdPlan plan_fwd(const Shape& s, int causal, kata_feature_t f = KATA_FEATURE_PSD,
                 kata_prefix_t pf = KATA_PREFIX_SCAN, int seg_req = 0) {
    FwdPlan p{};
    if (f == KATA_FEATURE_IDENTITY) {
        // matrix cores for the bf16 shapes, else the fp32 path (scan prefix)
        p.mfma = kata::first_supported(s) ? 1 : 0;
        p.ok = p.mfma != 0 || pf != KATA_PREFIX_SEQUENTIAL;
    } else {
        p.mfma = kata::mfma16_supported(s) ? 16 : kata::mfma32_supported(s) ? 32 : 0;
        p.ok = p.mfma != 0 || pf != KATA_PREFIX_SEQUENTIAL;
    }
    p.seq = pf == KATA_PREFIX_SEQUENTIAL;
    p.tree = pf == KATA_PREFIX_TREE;
    const size_t BH = (size_t)s.B * s.H;
    if (!p.ok || BH == 0 || s.NC == 0) return p;
    if (p.mfma) {
        // d_k = 16 and the identity feature: four 2-wavefront workgroups per
        // compute unit; d_k = 32: one workgroup (its LDS fills the compute unit)
        p.G = p.seq ? s.NC : std::min(segment_chunks(s, p.mfma == 32 ? 256 : 1024, seg_req), s.NC);
        p.NSEG = (s.NC + p.G - 1) / p.G;
        p.REC = p.mfma == 16   ? kata::mfma16_record_floats(s.dv)
                : p.mfma == 32 ? kata::mfma32_record_floats(s.dv)
                               : kata::first_record_floats(s.dk, s.dv);
        p.S_off = 0;
        p.init_off = align256(BH * p.NSEG * p.REC * sizeof(float));
        p.total_off = p.init_off + align256(BH * p.REC * sizeof(float));
        p.tree_off = p.total_off + align256(BH * p.REC * sizeof(float));
        // the tree scan's tile sums (and, gated, tile and record decays)
        const size_t tree = p.tree ? kata::scan_tree_scratch_floats((int)BH, p.NSEG, p.REC, true) : 0;
        p.bytes = p.tree_off + align256(tree * sizeof(float));
        return p;
    }
    // non-causal also needs the per-chunk totals before reducing them
    const size_t nrec = BH * (size_t)s.NC + (causal ? 0 : BH);
    p.S_off = 0;
    p.z_off = align256(nrec * s.D * s.dv * sizeof(float));
    p.tree_off = p.z_off + align256(nrec * s.D * sizeof(float));
    const size_t tree = p.tree ? kata::scan_tree_scratch_floats((int)BH, s.NC, s.D * s.dv, true) : 0;
    p.bytes = p.tree_off + align256(tree * sizeof(float));
    return p;
}

kata_status_t hip_status(hipError_t e) { return e == hipSuccess ? KATA_OK : KATA_EHIP; }

}  // namespace

extern "C" {

int kata_phi_dim(int d) { return d < 0 ? -1 : d * (d + 1) / 2; }

const char* kata_status_string(kata_status_t st) {
    switch (st) {
        case KATA_OK: return "ok";
        case KATA_EINVAL: return "invalid argument";
        case KATA_EUNSUPPORTED: return "unsupported shape";
        case KATA_EWORKSPACE: return "workspace too small";
        case KATA_EHIP: return "HIP launch error";
        case KATA_ESCRATCH: return "problem needs more than the static scratch";
    }
    return "unknown status";
}

const char* kata_version(void) { return "0.2.0"; }

size_t kata_chunked_fwd_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                  kata_dtype_t dtype, int causal) {
    Shape s;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s) != KATA_OK) return 0;
    return plan_fwd(s, causal).bytes;
}

int kata_feature_dim(int d, kata_feature_t feature) {
    if (d < 0) return -1;
    if (feature == KATA_FEATURE_PSD) return d * (d + 1) / 2;
    if (feature == KATA_FEATURE_IDENTITY) return d;
    return -1;
}

static bool valid_modes(kata_feature_t f, kata_prefix_t pf) {
    return (f == KATA_FEATURE_PSD || f == KATA_FEATURE_IDENTITY) &&
           (pf == KATA_PREFIX_SCAN || pf == KATA_PREFIX_SEQUENTIAL || pf == KATA_PREFIX_TREE);
}

// The scan over n records by the plan's method (blocked or tree); dec: the
// per-record decays of the gated operator (NULL = plain addition).
static hipError_t scan_by_plan(const FwdPlan& p, char* ws, float* rec, const float* dec, int nseq,
                               int n, int E, const float* init, float* total_a, float* total_b,
                               hipStream_t hs, const kata::RecordExport* ex = nullptr) {
    if (p.tree)
        return kata::launch_scan_records_tree(rec, dec, nseq, n, E, init, total_a, total_b,
                                              reinterpret_cast<float*>(ws + p.tree_off), hs, ex);
    return dec ? kata::launch_scan_records_decay(rec, dec, nseq, n, E, init, total_a, total_b, hs, ex)
               : kata::launch_scan_records(rec, nseq, n, E, init, total_a, total_b, hs, ex);
}

int kata_prefix_depth(int B, int H, int T, int d_k, int d_v, int chunk, kata_dtype_t dtype,
                      kata_feature_t feature, kata_prefix_t prefix, int segment_chunks) {
    Shape s;
    if (!valid_modes(feature, prefix) || segment_chunks < 0) return -1;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s, feature) != KATA_OK) return -1;
    const FwdPlan p = plan_fwd(s, 1, feature, prefix, segment_chunks);
    if (!p.ok) return -1;
    if ((size_t)B * H == 0 || s.NC == 0) return 0;
    const int method = p.tree ? 2 : 0;
    if (!p.mfma) return kata::scan_levels(s.NC, method);
    if (p.seq) return s.NC;
    // a segment's chunks in order, after the scan over segment states
    return p.G + kata::scan_levels(p.NSEG, method);
}

size_t kata_chunked_fwd_ex_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                     kata_dtype_t dtype, int causal, kata_feature_t feature,
                                     kata_prefix_t prefix, int segment_chunks) {
    Shape s;
    if (!valid_modes(feature, prefix) || segment_chunks < 0) return 0;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s, feature) != KATA_OK) return 0;
    return plan_fwd(s, causal, feature, prefix, segment_chunks).bytes;
}

static kata_status_t chunked_fwd_impl(const void* q, const void* k, const void* v, void* o,
                                      int B, int H, int T, int d_k, int d_v, int chunk,
                                      int causal, kata_dtype_t dtype, kata_feature_t feature,
                                      kata_prefix_t prefix, int seg_req, const float* S0,
                                      const float* z0, float* S_out, float* z_out,
                                      void* workspace, size_t ws_bytes, void* stream,
                                      void* const* events) {
    Shape s;
    if (!valid_modes(feature, prefix) || seg_req < 0) return KATA_EINVAL;
    kata_status_t st = make_shape(B, H, T, d_k, d_v, chunk, dtype, &s, feature);
    if (st != KATA_OK) return st;
    if ((S0 == nullptr) != (z0 == nullptr)) return KATA_EINVAL;
    if ((S_out == nullptr) != (z_out == nullptr)) return KATA_EINVAL;
    const size_t BH = (size_t)B * H;
    const bool empty = BH == 0 || T == 0;
    if (!empty && (!q || !k || !v || !o)) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)o,
                          (const void*)S0, (const void*)z0, (const void*)S_out,
                          (const void*)z_out, (const void*)workspace})
        if (p && !aligned16(p)) return KATA_EINVAL;
    const FwdPlan plan = plan_fwd(s, causal, feature, prefix, seg_req);
    if (!plan.ok) return KATA_EUNSUPPORTED;
    if (ws_bytes < plan.bytes || (plan.bytes && !workspace)) return KATA_EWORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t nS = (size_t)s.D * s.dv, nz = s.D;
    auto mark = [&](int i) -> hipError_t {
        return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), hs) : hipSuccess;
    };

    if (empty) {
        hipError_t e = mark(0);
        if (e == hipSuccess) e = mark(1);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) e = mark(3);
        if (S_out) {
            if (e == hipSuccess) e = kata::launch_copy_or_zero(S_out, S0, BH * nS, hs);
            if (e == hipSuccess) e = kata::launch_copy_or_zero(z_out, z0, BH * nz, hs);
        }
        if (e == hipSuccess) e = mark(4);
        return hip_status(e);
    }

    char* ws = static_cast<char*>(workspace);
    hipError_t e = mark(0);
    if (plan.mfma) {
        float* rec = reinterpret_cast<float*>(ws + plan.S_off);
        float* init = reinterpret_cast<float*>(ws + plan.init_off);
        float* total = reinterpret_cast<float*>(ws + plan.total_off);
        const int m = plan.mfma, nrec = (int)BH;
        auto from_packed = [&]() {
            return m == 16   ? kata::launch_record_from_packed16(init, S0, z0, s.dv, nrec, hs)
                   : m == 32 ? kata::launch_record_from_packed32(init, S0, z0, s.dv, nrec, hs)
                             : kata::launch_record_from_packed1(init, S0, z0, s.dk, s.dv, nrec, hs);
        };
        auto to_packed = [&]() {
            return m == 16   ? kata::launch_record_to_packed16(total, S_out, z_out, s.dv, nrec, hs)
                   : m == 32 ? kata::launch_record_to_packed32(total, S_out, z_out, s.dv, nrec, hs)
                             : kata::launch_record_to_packed1(total, S_out, z_out, s.dk, s.dv, nrec, hs);
        };
        // An initial state may stand for only a few tokens. Where it is the
        // whole inter-chunk prefix - the first chunk of every head - or, with
        // the keys of one chunk, the whole non-causal state, the output would
        // carry the bf16 rounding of lifted queries, keys, state entries and
        // the Gram matrix (terms of size |q|^2 |k|^2 summing to (q.k)^2)
        // un-averaged. Those chunks are evaluated with split (hi + lo)
        // operands; every later chunk's prefix also holds at least one whole
        // chunk of keys.
        const bool prec_all = S0 && !causal && s.NC == 1;
        auto seg_state = [&]() {
            return m == 16   ? kata::launch_seg_state16(s, k, v, rec, plan.G, plan.NSEG, prec_all, hs)
                   : m == 32 ? kata::launch_seg_state32(s, k, v, rec, plan.G, plan.NSEG, prec_all, hs)
                             : kata::launch_seg_state1(s, k, v, rec, plan.G, plan.NSEG, hs);
        };
        auto output = [&](const float* pre, float* fin) {
            return m == 16   ? kata::launch_fwd16(s, q, k, v, pre, fin, o, causal, plan.G, plan.NSEG, prec_all, hs)
                   : m == 32 ? kata::launch_fwd32(s, q, k, v, pre, fin, o, causal, plan.G, plan.NSEG, prec_all, hs)
                             : kata::launch_fwd1(s, q, k, v, pre, fin, o, causal, plan.G, plan.NSEG, hs,
                                                 plan.seq);
        };
        // the first chunk of every head again, from the initial-state record
        // (one segment of one chunk per head; the output launch above wrote it
        // with plain operands first)
        auto first_chunk_split = [&]() {
            if (m == 1 || !S0 || !causal) return hipSuccess;
            return m == 16 ? kata::launch_fwd16(s, q, k, v, init, nullptr, o, 1, 1, 1, true, hs)
                           : kata::launch_fwd32(s, q, k, v, init, nullptr, o, 1, 1, 1, true, hs);
        };
        if (S0 && e == hipSuccess) e = from_packed();
        if (plan.seq && causal) {
            // one segment per head walks every chunk from the initial state; its
            // running state at the end is the final state (the first-order
            // feature splits the walk over 16-column value tiles, one
            // workgroup each, so that it is not held to B*H workgroups)
            if (!S0 && e == hipSuccess)
                e = kata::launch_copy_or_zero(init, nullptr, BH * plan.REC, hs);
            if (e == hipSuccess) e = mark(1);
            if (e == hipSuccess) e = mark(2);
            if (e == hipSuccess) e = output(init, S_out ? total : nullptr);
            if (e == hipSuccess) e = first_chunk_split();
            if (e == hipSuccess) e = mark(3);
            if (S_out && e == hipSuccess) e = to_packed();
        } else {
            // Non-causal within one chunk and without an initial state: the
            // quadratic form gives o with every (q.k)^2 formed in fp32. Through
            // the total state each weight would carry the absolute error of the
            // bf16 lifted features (about 2^-9 |q|^2 |k|^2), which a few keys
            // with small (q.k)^2 do not average out. The final state, when asked
            // for, still comes from the segment state and the scan.
            const bool quad = !causal && !S0 && s.NC == 1 && m != 1 && kata::flash_supported(s);
            if (!quad || S_out) {
                if (e == hipSuccess) e = seg_state();
                if (e == hipSuccess) e = mark(1);
                // exclusive prefix over segments in place; the inclusive total
                // per head goes to the packed final state (when asked for) and,
                // for the non-causal output, to the total record
                const kata::RecordExport ex{m == 16 ? kata::kRecPsd16 : m == 32 ? kata::kRecPsd32
                                                                                : kata::kRecIdent,
                                            s.dk, s.dv, S_out, z_out};
                if (e == hipSuccess)
                    e = scan_by_plan(plan, ws, rec, nullptr, (int)BH, plan.NSEG, plan.REC,
                                     S0 ? init : nullptr, causal ? nullptr : total, nullptr, hs,
                                     S_out ? &ex : nullptr);
            } else if (e == hipSuccess) {
                e = mark(1);
            }
            if (e == hipSuccess) e = mark(2);
            if (e == hipSuccess)
                e = quad ? kata::launch_flash_fwd(s, q, k, v, o, 0, hs) : output(causal ? rec : total, nullptr);
            if (e == hipSuccess) e = first_chunk_split();
            if (e == hipSuccess) e = mark(3);
        }
        if (e == hipSuccess) e = mark(4);
        return hip_status(e);
    }
    float* S_rec = reinterpret_cast<float*>(ws + plan.S_off);
    float* z_rec = reinterpret_cast<float*>(ws + plan.z_off);
    const int ident = feature == KATA_FEATURE_IDENTITY;
    if (e == hipSuccess)
        e = kata::launch_chunk_states_valu(s, k, v, nullptr, S_rec, z_rec, nullptr, ident, hs);
    if (e == hipSuccess) e = mark(1);
    if (causal) {
        // exclusive prefix over chunks in place; inclusive total -> final state
        if (e == hipSuccess)
            e = scan_by_plan(plan, ws, S_rec, nullptr, (int)BH, s.NC, (int)nS, S0, S_out, nullptr, hs);
        if (e == hipSuccess)
            e = scan_by_plan(plan, ws, z_rec, nullptr, (int)BH, s.NC, (int)nz, z0, z_out, nullptr, hs);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) e = kata::launch_fwd_valu(s, q, k, v, nullptr, S_rec, z_rec, o, 1, ident, hs);
    } else {
        // total state per head, stored after the per-chunk records
        float* S_tot = S_rec + BH * s.NC * nS;
        float* z_tot = z_rec + BH * s.NC * nz;
        if (e == hipSuccess)
            e = scan_by_plan(plan, ws, S_rec, nullptr, (int)BH, s.NC, (int)nS, S0, S_tot, S_out, hs);
        if (e == hipSuccess)
            e = scan_by_plan(plan, ws, z_rec, nullptr, (int)BH, s.NC, (int)nz, z0, z_tot, z_out, hs);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) e = kata::launch_fwd_valu(s, q, k, v, nullptr, S_tot, z_tot, o, 0, ident, hs);
    }
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = mark(4);
    return hip_status(e);
}

kata_status_t kata_chunked_fwd(const void* q, const void* k, const void* v, void* o,
                               int B, int H, int T, int d_k, int d_v, int chunk, int causal,
                               kata_dtype_t dtype, const float* S0, const float* z0,
                               float* S_out, float* z_out, void* workspace, size_t ws_bytes,
                               void* stream) {
    return chunked_fwd_impl(q, k, v, o, B, H, T, d_k, d_v, chunk, causal, dtype, KATA_FEATURE_PSD,
                            KATA_PREFIX_SCAN, 0, S0, z0, S_out, z_out, workspace, ws_bytes, stream,
                            nullptr);
}

kata_status_t kata_chunked_fwd_ex(const void* q, const void* k, const void* v, void* o, int B,
                                  int H, int T, int d_k, int d_v, int chunk, int causal,
                                  kata_dtype_t dtype, kata_feature_t feature,
                                  kata_prefix_t prefix, int segment_chunks, const float* S0,
                                  const float* z0, float* S_out, float* z_out, void* workspace,
                                  size_t ws_bytes, void* stream) {
    return chunked_fwd_impl(q, k, v, o, B, H, T, d_k, d_v, chunk, causal, dtype, feature, prefix,
                            segment_chunks, S0, z0, S_out, z_out, workspace, ws_bytes, stream,
                            nullptr);
}

kata_status_t kata_chunked_fwd_profiled(const void* q, const void* k, const void* v, void* o,
                                        int B, int H, int T, int d_k, int d_v, int chunk,
                                        int causal, kata_dtype_t dtype, const float* S0,
                                        const float* z0, float* S_out, float* z_out,
                                        void* workspace, size_t ws_bytes, void* stream,
                                        void* const* events, int n_events) {
    if (!events || n_events < 5) return KATA_EINVAL;
    for (int i = 0; i < 5; ++i)
        if (!events[i]) return KATA_EINVAL;
    return chunked_fwd_impl(q, k, v, o, B, H, T, d_k, d_v, chunk, causal, dtype, KATA_FEATURE_PSD,
                            KATA_PREFIX_SCAN, 0, S0, z0, S_out, z_out, workspace, ws_bytes, stream,
                            events);
}

// kata_scan_states on the matrix cores (bf16, PSD shapes of the output
// kernels): segment states with split key operands, the scan over segment
// records (the initial state as its identity, the packed total as S_out), then
// each segment's chunks walked from its prefix, every chunk's exclusive prefix
// written in the packed layout. Workspace: the segment records and one
// initial-state record per head.
static FwdPlan scan_plan(const Shape& s) {
    FwdPlan p = plan_fwd(s, 1);
    if (!p.mfma) p.bytes = 0;                 // the fp32 path writes into S_prefix itself
    else p.bytes = p.total_off;               // no final-state record
    return p;
}

size_t kata_scan_states_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                  kata_dtype_t dtype) {
    Shape s;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s) != KATA_OK) return 0;
    return scan_plan(s).bytes;
}

kata_status_t kata_scan_states(const void* k, const void* v, int B, int H, int T, int d_k,
                               int d_v, int chunk, kata_dtype_t dtype, const float* S0,
                               const float* z0, float* S_prefix, float* z_prefix, float* S_out,
                               float* z_out, void* workspace, size_t ws_bytes, void* stream) {
    Shape s;
    kata_status_t st = make_shape(B, H, T, d_k, d_v, chunk, dtype, &s);
    if (st != KATA_OK) return st;
    if ((S0 == nullptr) != (z0 == nullptr)) return KATA_EINVAL;
    if ((S_out == nullptr) != (z_out == nullptr)) return KATA_EINVAL;
    const size_t BH = (size_t)B * H;
    const bool empty = BH == 0 || T == 0;
    if (!empty && (!k || !v || !S_prefix || !z_prefix)) return KATA_EINVAL;
    for (const void* p : {(const void*)k, (const void*)v, (const void*)S0, (const void*)z0,
                          (const void*)S_prefix, (const void*)z_prefix, (const void*)S_out,
                          (const void*)z_out, (const void*)workspace})
        if (p && !aligned16(p)) return KATA_EINVAL;
    const FwdPlan plan = empty ? FwdPlan{} : scan_plan(s);
    if (ws_bytes < plan.bytes || (plan.bytes && !workspace)) return KATA_EWORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t nS = (size_t)s.D * s.dv, nz = s.D;
    if (empty) {
        if (S_out) {
            hipError_t e = kata::launch_copy_or_zero(S_out, S0, BH * nS, hs);
            if (e == hipSuccess) e = kata::launch_copy_or_zero(z_out, z0, BH * nz, hs);
            return hip_status(e);
        }
        return KATA_OK;
    }
    if (plan.mfma == 16 || plan.mfma == 32) {
        char* ws = static_cast<char*>(workspace);
        float* rec = reinterpret_cast<float*>(ws + plan.S_off);
        float* init = reinterpret_cast<float*>(ws + plan.init_off);
        const bool m16 = plan.mfma == 16;
        hipError_t e = hipSuccess;
        if (S0)
            e = m16 ? kata::launch_record_from_packed16(init, S0, z0, s.dv, (int)BH, hs)
                    : kata::launch_record_from_packed32(init, S0, z0, s.dv, (int)BH, hs);
        if (e == hipSuccess)
            e = m16 ? kata::launch_seg_state16(s, k, v, rec, plan.G, plan.NSEG, true, hs)
                    : kata::launch_seg_state32(s, k, v, rec, plan.G, plan.NSEG, true, hs);
        const kata::RecordExport ex{m16 ? kata::kRecPsd16 : kata::kRecPsd32, s.dk, s.dv, S_out, z_out};
        if (e == hipSuccess)
            e = kata::launch_scan_records(rec, (int)BH, plan.NSEG, plan.REC, S0 ? init : nullptr,
                                          nullptr, nullptr, hs, S_out ? &ex : nullptr);
        if (e == hipSuccess)
            e = m16 ? kata::launch_prefix16(s, k, v, rec, S_prefix, z_prefix, plan.G, plan.NSEG, hs)
                    : kata::launch_prefix32(s, k, v, rec, S_prefix, z_prefix, plan.G, plan.NSEG, hs);
        return hip_status(e);
    }
    hipError_t e = kata::launch_chunk_states_valu(s, k, v, nullptr, S_prefix, z_prefix, nullptr, 0, hs);
    if (e == hipSuccess)
        e = kata::launch_scan_records(S_prefix, (int)BH, s.NC, (int)nS, S0, S_out, nullptr, hs);
    if (e == hipSuccess)
        e = kata::launch_scan_records(z_prefix, (int)BH, s.NC, (int)nz, z0, z_out, nullptr, hs);
    return hip_status(e);
}

kata_status_t kata_flash_fwd(const void* q, const void* k, const void* v, void* o, int B, int H,
                             int T, int d_k, int d_v, int causal, kata_dtype_t dtype,
                             void* stream) {
    Shape s;
    // the chunk size does not enter the quadratic form; any supported value
    kata_status_t st = make_shape(B, H, T, d_k, d_v, 64, dtype, &s);
    if (st != KATA_OK) return st;
    if (!kata::flash_supported(s)) return KATA_EUNSUPPORTED;
    if ((size_t)B * H == 0 || T == 0) return KATA_OK;
    if (!q || !k || !v || !o) return KATA_EINVAL;
    for (const void* p : {q, k, v, (const void*)o})
        if (!aligned16(p)) return KATA_EINVAL;
    return hip_status(kata::launch_flash_fwd(s, q, k, v, o, causal, static_cast<hipStream_t>(stream)));
}

// ---- decay gate ----------------------------------------------------------------

// Matrix-core paths (segments, scan or sequential prefix): the PSD lift for
// bf16 at d_k = 16 (C 32 or 64) and d_k = 32 (C 64 or 128), the identity
// feature for bf16 with C 32 or 64. They stage each chunk's log-decays 16 bytes
// at a time from T-aligned offsets, so with several heads T must be a multiple
// of 4. Every other case takes the fp32 path (per-chunk records, scan
// prefix only).
struct DecayPlan {
    FwdPlan fwd;           // matrix-core path
    bool valu = false;     // VALU path: S_rec | z_rec | cdec, one record per chunk
    size_t z_off = 0, dec_off = 0, bytes = 0;
};

static bool decay_plan(const Shape& s, kata_feature_t f, kata_prefix_t prefix, int seg_req,
                       DecayPlan* d) {
    const size_t BH = (size_t)s.B * s.H;
    const bool aligned_rows = s.T % 4 == 0 || BH <= 1;
    if (aligned_rows &&
        ((f == KATA_FEATURE_PSD && (kata::mfma16_supported(s) || kata::mfma32_supported(s))) ||
         (f == KATA_FEATURE_IDENTITY && kata::first_decay_supported(s)))) {
        d->fwd = plan_fwd(s, 1, f, prefix, seg_req);
        if (!d->fwd.ok) return false;
        d->dec_off = d->fwd.bytes;
        d->bytes = d->fwd.bytes;
        if (!d->fwd.seq) d->bytes += align256(BH * d->fwd.NSEG * sizeof(float));
        return true;
    }
    if (prefix != KATA_PREFIX_SCAN) return BH * s.NC == 0;   // nothing to run when empty
    const size_t nrec = BH * s.NC;
    d->valu = true;
    d->z_off = align256(nrec * s.D * s.dv * sizeof(float));
    d->dec_off = d->z_off + align256(nrec * s.D * sizeof(float));
    d->bytes = nrec ? d->dec_off + align256(nrec * sizeof(float)) : 0;
    return true;
}

size_t kata_chunked_fwd_decay_ex_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                           kata_dtype_t dtype, kata_feature_t feature,
                                           kata_prefix_t prefix, int segment_chunks) {
    Shape s;
    DecayPlan p;
    if (!valid_modes(feature, prefix) || segment_chunks < 0) return 0;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s, feature) != KATA_OK) return 0;
    if (!decay_plan(s, feature, prefix, segment_chunks, &p)) return 0;
    return p.bytes;
}

size_t kata_chunked_fwd_decay_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                        kata_dtype_t dtype, kata_prefix_t prefix) {
    return kata_chunked_fwd_decay_ex_workspace(B, H, T, d_k, d_v, chunk, dtype, KATA_FEATURE_PSD,
                                               prefix, 0);
}

kata_status_t kata_chunked_fwd_decay_ex(const void* q, const void* k, const void* v,
                                        const float* log_decay, void* o, int B, int H, int T,
                                        int d_k, int d_v, int chunk, kata_dtype_t dtype,
                                        kata_feature_t feature, kata_prefix_t prefix,
                                        int segment_chunks, const float* S0, const float* z0,
                                        float* S_out, float* z_out, void* workspace,
                                        size_t ws_bytes, void* stream) {
    if (!valid_modes(feature, prefix) || segment_chunks < 0) return KATA_EINVAL;
    Shape s;
    kata_status_t st = make_shape(B, H, T, d_k, d_v, chunk, dtype, &s, feature);
    if (st != KATA_OK) return st;
    if ((S0 == nullptr) != (z0 == nullptr)) return KATA_EINVAL;
    if ((S_out == nullptr) != (z_out == nullptr)) return KATA_EINVAL;
    const size_t BH = (size_t)B * H;
    const bool empty = BH == 0 || T == 0;
    if (!empty && (!q || !k || !v || !o || !log_decay)) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)o,
                          (const void*)log_decay, (const void*)S0, (const void*)z0,
                          (const void*)S_out, (const void*)z_out, (const void*)workspace})
        if (p && !aligned16(p)) return KATA_EINVAL;
    DecayPlan plan;
    if (!decay_plan(s, feature, prefix, segment_chunks, &plan)) return KATA_EUNSUPPORTED;
    if (ws_bytes < plan.bytes || (plan.bytes && !workspace)) return KATA_EWORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t nS = (size_t)s.D * s.dv, nz = s.D;
    if (empty) {
        hipError_t e = hipSuccess;
        if (S_out) {
            e = kata::launch_copy_or_zero(S_out, S0, BH * nS, hs);
            if (e == hipSuccess) e = kata::launch_copy_or_zero(z_out, z0, BH * nz, hs);
        }
        return hip_status(e);
    }
    char* ws = static_cast<char*>(workspace);
    hipError_t e = hipSuccess;
    if (plan.valu) {
        const int ident = feature == KATA_FEATURE_IDENTITY;
        float* S_rec = reinterpret_cast<float*>(ws);
        float* z_rec = reinterpret_cast<float*>(ws + plan.z_off);
        float* cdec = reinterpret_cast<float*>(ws + plan.dec_off);
        e = kata::launch_chunk_states_valu(s, k, v, log_decay, S_rec, z_rec, cdec, ident, hs);
        // exclusive prefix over chunks under the decayed combine; inclusive
        // total -> final state
        if (e == hipSuccess)
            e = kata::launch_scan_records_decay(S_rec, cdec, (int)BH, s.NC, (int)nS, S0, S_out,
                                                nullptr, hs);
        if (e == hipSuccess)
            e = kata::launch_scan_records_decay(z_rec, cdec, (int)BH, s.NC, (int)nz, z0, z_out,
                                                nullptr, hs);
        if (e == hipSuccess)
            e = kata::launch_fwd_valu(s, q, k, v, log_decay, S_rec, z_rec, o, 1, ident, hs);
        return hip_status(e);
    }
    const FwdPlan& fp = plan.fwd;
    const int m = fp.mfma;                        // 1: identity feature; 16, 32: PSD lift at d_k
    float* rec = reinterpret_cast<float*>(ws + fp.S_off);
    float* init = reinterpret_cast<float*>(ws + fp.init_off);
    float* total = reinterpret_cast<float*>(ws + fp.total_off);
    const int nrec = (int)BH;
    auto output = [&](const float* pre, float* fin) {
        return m == 1    ? kata::launch_fwd1_decay(s, q, k, v, log_decay, pre, fin, o, fp.G, fp.NSEG, hs,
                                                   fp.seq)
               : m == 16 ? kata::launch_fwd16_decay(s, q, k, v, log_decay, pre, fin, o, fp.G, fp.NSEG, hs)
                         : kata::launch_fwd32_decay(s, q, k, v, log_decay, pre, fin, o, fp.G, fp.NSEG, hs);
    };
    if (S0)
        e = m == 1    ? kata::launch_record_from_packed1(init, S0, z0, s.dk, s.dv, nrec, hs)
            : m == 16 ? kata::launch_record_from_packed16(init, S0, z0, s.dv, nrec, hs)
                      : kata::launch_record_from_packed32(init, S0, z0, s.dv, nrec, hs);
    if (fp.seq) {
        if (!S0 && e == hipSuccess) e = kata::launch_copy_or_zero(init, nullptr, BH * fp.REC, hs);
        if (e == hipSuccess) e = output(init, S_out ? total : nullptr);
        if (S_out && e == hipSuccess)
            e = m == 1    ? kata::launch_record_to_packed1(total, S_out, z_out, s.dk, s.dv, nrec, hs)
                : m == 16 ? kata::launch_record_to_packed16(total, S_out, z_out, s.dv, nrec, hs)
                          : kata::launch_record_to_packed32(total, S_out, z_out, s.dv, nrec, hs);
    } else {
        float* segdec = reinterpret_cast<float*>(ws + plan.dec_off);
        const kata::RecordExport ex{m == 1 ? kata::kRecIdent : m == 16 ? kata::kRecPsd16 : kata::kRecPsd32,
                                    s.dk, s.dv, S_out, z_out};
        if (e == hipSuccess)
            e = m == 1    ? kata::launch_seg_state1_decay(s, k, v, log_decay, rec, segdec, fp.G, fp.NSEG, hs)
                : m == 16 ? kata::launch_seg_state16_decay(s, k, v, log_decay, rec, segdec, fp.G, fp.NSEG, hs)
                          : kata::launch_seg_state32_decay(s, k, v, log_decay, rec, segdec, fp.G, fp.NSEG, hs);
        if (e == hipSuccess)
            e = scan_by_plan(fp, ws, rec, segdec, nrec, fp.NSEG, fp.REC, S0 ? init : nullptr,
                             nullptr, nullptr, hs, S_out ? &ex : nullptr);
        if (e == hipSuccess) e = output(rec, nullptr);
    }
    return hip_status(e);
}

kata_status_t kata_chunked_fwd_decay(const void* q, const void* k, const void* v,
                                     const float* log_decay, void* o, int B, int H, int T,
                                     int d_k, int d_v, int chunk, kata_dtype_t dtype,
                                     kata_prefix_t prefix, const float* S0, const float* z0,
                                     float* S_out, float* z_out, void* workspace, size_t ws_bytes,
                                     void* stream) {
    return kata_chunked_fwd_decay_ex(q, k, v, log_decay, o, B, H, T, d_k, d_v, chunk, dtype,
                                     KATA_FEATURE_PSD, prefix, 0, S0, z0, S_out, z_out, workspace,
                                     ws_bytes, stream);
}

kata_status_t kata_decode_step_decay(const void* q, const void* k, const void* v,
                                     const float* log_decay, float* S, float* z, void* o, int N,
                                     int d_k, int d_v, kata_dtype_t dtype, void* stream) {
    if (N < 0 || d_k < 0 || d_v < 0) return KATA_EINVAL;
    if (dtype != KATA_F32 && dtype != KATA_BF16) return KATA_EINVAL;
    if (!supported_dk(d_k) || !supported_dv(d_v)) return KATA_EUNSUPPORTED;
    if (N == 0) return KATA_OK;
    if (!q || !k || !v || !S || !z || !o || !log_decay) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)S,
                          (const void*)z, (const void*)o, (const void*)log_decay})
        if (!aligned16(p)) return KATA_EINVAL;
    return hip_status(kata::launch_decode(q, k, v, log_decay, S, z, o, N, d_k, d_v,
                                          dtype == KATA_BF16, static_cast<hipStream_t>(stream)));
}

kata_status_t kata_decode_step(const void* q, const void* k, const void* v, float* S, float* z,
                               void* o, int N, int d_k, int d_v, kata_dtype_t dtype,
                               void* stream) {
    if (N < 0 || d_k < 0 || d_v < 0) return KATA_EINVAL;
    if (dtype != KATA_F32 && dtype != KATA_BF16) return KATA_EINVAL;
    if (!supported_dk(d_k) || !supported_dv(d_v)) return KATA_EUNSUPPORTED;
    if (N == 0) return KATA_OK;
    if (!q || !k || !v || !S || !z || !o) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)S,
                          (const void*)z, (const void*)o})
        if (!aligned16(p)) return KATA_EINVAL;
    return hip_status(kata::launch_decode(q, k, v, nullptr, S, z, o, N, d_k, d_v,
                                          dtype == KATA_BF16, static_cast<hipStream_t>(stream)));
}

// ---- DeltaKATA ---------------------------------------------------------------

size_t kata_delta_fwd_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                kata_dtype_t dtype) {
    Shape s;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s) != KATA_OK || !kata::delta_supported(s))
        return 0;
    return kata::delta_workspace_bytes(s);
}

kata_status_t kata_delta_fwd(const void* q, const void* k, const void* v, const float* beta,
                             void* o, int B, int H, int T, int d_k, int d_v, int chunk,
                             kata_dtype_t dtype, const float* S0, const float* z0, float* S_out,
                             float* z_out, void* workspace, size_t ws_bytes, void* stream) {
    Shape s;
    kata_status_t st = make_shape(B, H, T, d_k, d_v, chunk, dtype, &s);
    if (st != KATA_OK) return st;
    if (!kata::delta_supported(s)) return KATA_EUNSUPPORTED;
    if ((S0 == nullptr) != (z0 == nullptr)) return KATA_EINVAL;
    if ((S_out == nullptr) != (z_out == nullptr)) return KATA_EINVAL;
    const size_t BH = (size_t)B * H;
    const bool empty = BH == 0 || T == 0;
    if (!empty && (!q || !k || !v || !o || !beta)) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)o,
                          (const void*)beta, (const void*)S0, (const void*)z0, (const void*)S_out,
                          (const void*)z_out, (const void*)workspace})
        if (p && !aligned16(p)) return KATA_EINVAL;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (empty) {
        hipError_t e = hipSuccess;
        if (S_out) {
            e = kata::launch_copy_or_zero(S_out, S0, BH * s.D * s.dv, hs);
            if (e == hipSuccess) e = kata::launch_copy_or_zero(z_out, z0, BH * s.D, hs);
        }
        return hip_status(e);
    }
    if (!workspace || ws_bytes < kata::delta_workspace_bytes(s)) return KATA_EWORKSPACE;
    return hip_status(kata::launch_delta_fwd(s, q, k, v, beta, o, S0, z0, S_out, z_out,
                                             static_cast<float*>(workspace), hs));
}

kata_status_t kata_decode_step_delta(const void* q, const void* k, const void* v,
                                     const float* beta, float* S, float* z, void* o, int N,
                                     int d_k, int d_v, kata_dtype_t dtype, void* stream) {
    if (N < 0 || d_k < 0 || d_v < 0) return KATA_EINVAL;
    if (dtype != KATA_F32 && dtype != KATA_BF16) return KATA_EINVAL;
    if (!supported_dk(d_k) || !supported_dv(d_v)) return KATA_EUNSUPPORTED;
    if (N == 0) return KATA_OK;
    if (!q || !k || !v || !S || !z || !o || !beta) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)S,
                          (const void*)z, (const void*)o, (const void*)beta})
        if (!aligned16(p)) return KATA_EINVAL;
    return hip_status(kata::launch_delta_decode(q, k, v, beta, S, z, o, N, d_k, d_v,
                                                dtype == KATA_BF16, static_cast<hipStream_t>(stream)));
}

// ---- factored PSD features (KATA-Mg, KATA-Sigma-g) ----------------------------

}  // extern "C"

namespace {

// Workspace of kata_factored_fwd: segment records [BH, NSEG, REC], then the
// initial-state record and the total record per head (records in the
// first-order layout with the factored feature's rows).
struct FactPlan {
    bool ok;
    int G, NSEG, REC, D;
    size_t init_off, total_off, bytes;
};

FactPlan plan_fact(const Shape& s, int g, bool summed) {
    FactPlan p{};
    p.ok = kata::factored_supported(s, g, summed);
    const size_t BH = (size_t)s.B * s.H;
    if (!p.ok || BH == 0 || s.NC == 0) return p;
    p.D = kata::factored_dim(s.dk, g, summed);
    // four-wavefront workgroups, about two per compute unit
    p.G = std::min(segment_chunks(s, 512, 0), s.NC);
    p.NSEG = (s.NC + p.G - 1) / p.G;
    p.REC = kata::factored_record_floats(s.dk, s.dv, g, summed);
    p.init_off = align256(BH * p.NSEG * p.REC * sizeof(float));
    p.total_off = p.init_off + align256(BH * p.REC * sizeof(float));
    p.bytes = p.total_off + align256(BH * p.REC * sizeof(float));
    return p;
}

bool valid_factors(int g, kata_factors_t kind) {
    return g >= 1 && (kind == KATA_FACTORS_MULTI || kind == KATA_FACTORS_SUMMED);
}

}  // namespace

extern "C" {

int kata_factored_dim(int d, int g, kata_factors_t kind) {
    if (d < 0 || !valid_factors(g, kind) || d % g) return -1;
    return kata::factored_dim(d, g, kind == KATA_FACTORS_SUMMED);
}

size_t kata_factored_fwd_workspace(int B, int H, int T, int d_k, int d_v, int chunk,
                                   kata_dtype_t dtype, int causal, int g, kata_factors_t kind) {
    if (!valid_factors(g, kind)) return 0;
    if (g == 1) return kata_chunked_fwd_workspace(B, H, T, d_k, d_v, chunk, dtype, causal);
    Shape s;
    if (make_shape(B, H, T, d_k, d_v, chunk, dtype, &s) != KATA_OK || d_k % g) return 0;
    return plan_fact(s, g, kind == KATA_FACTORS_SUMMED).bytes;
}

kata_status_t kata_factored_fwd(const void* q, const void* k, const void* v, void* o, int B,
                                int H, int T, int d_k, int d_v, int chunk, int causal,
                                kata_dtype_t dtype, int g, kata_factors_t kind, const float* S0,
                                const float* z0, float* S_out, float* z_out, void* workspace,
                                size_t ws_bytes, void* stream) {
    if (!valid_factors(g, kind)) return KATA_EINVAL;
    if (g == 1)
        return kata_chunked_fwd(q, k, v, o, B, H, T, d_k, d_v, chunk, causal, dtype, S0, z0, S_out,
                                z_out, workspace, ws_bytes, stream);
    Shape s;
    kata_status_t st = make_shape(B, H, T, d_k, d_v, chunk, dtype, &s);
    if (st != KATA_OK) return st;
    if (d_k % g) return KATA_EINVAL;
    const bool summed = kind == KATA_FACTORS_SUMMED;
    s.D = kata::factored_dim(d_k, g, summed);
    if ((S0 == nullptr) != (z0 == nullptr)) return KATA_EINVAL;
    if ((S_out == nullptr) != (z_out == nullptr)) return KATA_EINVAL;
    const size_t BH = (size_t)B * H;
    const bool empty = BH == 0 || T == 0;
    if (!empty && (!q || !k || !v || !o)) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)o,
                          (const void*)S0, (const void*)z0, (const void*)S_out,
                          (const void*)z_out, (const void*)workspace})
        if (p && !aligned16(p)) return KATA_EINVAL;
    const FactPlan plan = plan_fact(s, g, summed);
    if (!plan.ok) return KATA_EUNSUPPORTED;
    if (ws_bytes < plan.bytes || (plan.bytes && !workspace)) return KATA_EWORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t nS = (size_t)s.D * s.dv, nz = s.D;
    if (empty) {
        hipError_t e = hipSuccess;
        if (S_out) {
            e = kata::launch_copy_or_zero(S_out, S0, BH * nS, hs);
            if (e == hipSuccess) e = kata::launch_copy_or_zero(z_out, z0, BH * nz, hs);
        }
        return hip_status(e);
    }
    char* ws = static_cast<char*>(workspace);
    float* rec = reinterpret_cast<float*>(ws);
    float* init = reinterpret_cast<float*>(ws + plan.init_off);
    float* total = reinterpret_cast<float*>(ws + plan.total_off);
    hipError_t e = hipSuccess;
    if (S0) e = kata::launch_fact_record_from_packed(init, S0, z0, s.D, s.dv, plan.REC, (int)BH, hs);
    if (e == hipSuccess)
        e = kata::launch_fact_seg_state(s, g, summed, k, v, rec, plan.G, plan.NSEG, hs);
    // exclusive prefix over segments in place; the inclusive total goes to the
    // packed final state (when asked for) and, for the non-causal output, to
    // the total record
    const kata::RecordExport ex{kata::kRecIdent, s.D, s.dv, S_out, z_out};
    if (e == hipSuccess)
        e = kata::launch_scan_records(rec, (int)BH, plan.NSEG, plan.REC, S0 ? init : nullptr,
                                      causal ? nullptr : total, nullptr, hs, S_out ? &ex : nullptr);
    if (e == hipSuccess)
        e = kata::launch_fact_fwd(s, g, summed, q, k, v, causal ? rec : total, o, causal, plan.G,
                                  plan.NSEG, hs);
    return hip_status(e);
}

kata_status_t kata_decode_step_factored(const void* q, const void* k, const void* v, float* S,
                                        float* z, void* o, int N, int d_k, int d_v, int g,
                                        kata_factors_t kind, kata_dtype_t dtype, void* stream) {
    if (N < 0 || d_k < 0 || d_v < 0 || !valid_factors(g, kind)) return KATA_EINVAL;
    if (dtype != KATA_F32 && dtype != KATA_BF16) return KATA_EINVAL;
    if (g == 1) return kata_decode_step(q, k, v, S, z, o, N, d_k, d_v, dtype, stream);
    if (d_k % g) return KATA_EINVAL;
    const bool summed = kind == KATA_FACTORS_SUMMED;
    if (!kata::factored_decode_supported(d_k, d_v, g, summed)) return KATA_EUNSUPPORTED;
    if (N == 0) return KATA_OK;
    if (!q || !k || !v || !S || !z || !o) return KATA_EINVAL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)S,
                          (const void*)z, (const void*)o})
        if (!aligned16(p)) return KATA_EINVAL;
    return hip_status(kata::launch_fact_decode(q, k, v, S, z, o, N, d_k, d_v, g, summed,
                                               dtype == KATA_BF16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- allocation-free forward ------------------------------------------------
// A file-scope device array stands in for the workspace. In host code its name
// is only a host-side handle: the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current, and
// only that address is ever passed to a kernel.

namespace {

static __device__ __align__(256) char scratch[KATA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch, or nullptr on failure.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
        g_scratch_ptr[dev].store(addr, std::memory_order_release);
        p = addr;
    }
    return p;
}

}  // namespace

extern "C" kata_status_t kata_chunked_fwd_noalloc(const void* q, const void* k, const void* v,
                                                  void* o, int B, int H, int T, int d_k, int d_v,
                                                  int chunk, int causal, kata_dtype_t dtype,
                                                  const float* S0, const float* z0,
                                                  float* S_out, float* z_out, void* stream) {
    Shape s;
    kata_status_t st = make_shape(B, H, T, d_k, d_v, chunk, dtype, &s);
    if (st != KATA_OK) return st;
    const size_t need = plan_fwd(s, causal).bytes;
    if (need > KATA_NOALLOC_SCRATCH_BYTES) return KATA_ESCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_for_current_device();
        if (!ws) return KATA_EHIP;
    }
    return chunked_fwd_impl(q, k, v, o, B, H, T, d_k, d_v, chunk, causal, dtype, KATA_FEATURE_PSD,
                            KATA_PREFIX_SCAN, 0, S0, z0, S_out, z_out, ws,
                            KATA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}
