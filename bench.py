"""Benchmark of the KATA chunked causal forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick [--workload W]]

A step is one pass of the whole hot path over the 131k-token workload (B1 H8
T131072 d_k16 d_v64 bf16, chunk 64, q/k unit-norm Gaussian rows, v ~ N(0,1)):
per-chunk or per-segment states, the associative scan over them, the fused
intra+inter output with normalisation, and the final-state export. Inputs are
resident in HBM before timing starts. The T=32k workload (B1 H16 d_k32 C128)
and 1024 decode steps on 512 x 4 rows are measured in the same run and
reported under "parts". Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KATA chunked fwd tokens/sec + MFMA util at T=32k/131k; decode HBM GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters_fwd131k.json")


# sources of the dominant (output) kernel: HBM counters taken on another build
# of it are not reported
DOMINANT_KERNEL_SOURCES = ("kata_fwd16.hip", "kata_chunk.h", "kata_mfma.h", "kata_device.h")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kernelized_linear_attention_phi_amd", "csrc")
    for name in DOMINANT_KERNEL_SOURCES:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def alg_flops_per_token_head(dk, dv, C):
    """QK^T, A.V, phi(K)^T V and phi(Q).P with dense C x C intra tiles."""
    D = dk * (dk + 1) // 2
    return 2 * C * dk + 2 * C * dv + 4 * D * dv


def alg_bytes_per_token_head(dk, dv, elem=2):
    """One read of q, k, v and one write of o."""
    return elem * (2 * dk + 2 * dv)


def time_forward(kata, torch, w, q, k, v, steps, warmup, sets=None):
    """Times `steps` forwards (state export included) with events on the stream
    the library launches on. Returns (ms per step, wall ms per step, per-phase
    ms): the per-step time comes from `steps` back-to-back forwards bracketed
    by one event pair; the phases from a second pass of `steps` forwards with
    events recorded between the phases (those events are instrumentation, so
    that pass is not the headline). sets: optional list of (q, k, v, o) input
    and output sets that step i rotates through (set i % len(sets)) instead of
    the one (q, k, v)."""
    B, H, T = w.B, w.H, w.T
    D = w.dk * (w.dk + 1) // 2
    if sets is None:
        sets = [(q, k, v, torch.empty_like(v))]
    S_out = torch.empty((B, H, D, w.dv), dtype=torch.float32, device="cuda")
    z_out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    nbytes = kata.chunked_fwd_workspace(B, H, T, w.dk, w.dv, w.chunk, 1, True)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def fwd(i, events=None):
        qi, ki, vi, oi = sets[i % len(sets)]
        kata.chunked_fwd_into(qi, ki, vi, oi, w.chunk, True, ws, S_out=S_out, z_out=z_out,
                              events=events)

    for i in range(warmup):
        fwd(i)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fwd(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    total = e0.elapsed_time(e1) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        fwd(i, evs[i])
    torch.cuda.synchronize()
    phases = {name: sum(evs[i][a].elapsed_time(evs[i][a + 1]) for i in range(steps)) / steps
              for a, name in enumerate(["states", "scan", "output", "export"])}
    phases["instrumented_total"] = sum(evs[i][0].elapsed_time(evs[i][4]) for i in range(steps)) / steps
    return total, wall, phases


def time_calls(torch, fn, steps, warmup):
    """Mean ms of fn() over `steps` calls, timed with events on the current stream."""
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def quadratic_vs_chunked(kata, torch, gen, name, steps, warmup):
    """The same workload through the chunked form and the quadratic form."""
    w = gen.WORKLOADS[name]
    q, k, v = gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype)
    to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    q, k, v = to(q), to(k), to(v)
    o = torch.empty_like(v)
    nbytes = kata.chunked_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1, True)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    ms_c = time_calls(torch, lambda: kata.chunked_fwd_into(q, k, v, o, w.chunk, True, ws),
                      steps, warmup)
    ms_f = time_calls(torch, lambda: kata.flash_fwd(q, k, v, out=o), steps, warmup)
    tok = w.B * w.T
    # quadratic form: 2 (d_k + d_v) flops per (query, key) pair, (T^2 + T) / 2 pairs
    qflops = w.B * w.H * (w.T * (w.T + 1) / 2) * 2 * (w.dk + w.dv)
    return {"chunked_ms": ms_c, "flash_ms": ms_f, "chunked_tokens_per_s": tok / (ms_c * 1e-3),
            "flash_tokens_per_s": tok / (ms_f * 1e-3),
            "flash_alg_tflops": qflops / (ms_f * 1e-3) / 1e12,
            "flash_mfma_util_alg": qflops / (ms_f * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def decode_bench(kata, torch, steps=1024, n_seq=512, heads=4, dk=16, dv=64, reps=3, gated=False):
    """`steps` decode steps on n_seq x heads rows with fp32 state, replayed from
    a HIP graph; returns ms per step and algorithmic GB/s. gated: the
    decay-gated step, with per-row log-decays in [-0.05, 0]. With 512 x 4 rows
    the state (72.4 MB) fits the 256 MB memory-side cache; with 2048 x 4 rows
    (290 MB) it does not, so every step streams it from DRAM."""
    from kernelized_linear_attention_phi_amd import inputs as gen
    N = n_seq * heads
    D = dk * (dk + 1) // 2
    rng = np.random.Generator(np.random.PCG64(5))
    q, k, _ = gen.gaussian_qkv(1, steps, N, dk, 1, seed=5000, dtype="bf16")
    vid = rng.integers(0, dv, (steps, N))
    v = np.zeros((steps, N, dv), dtype=np.float32)
    v[np.arange(steps)[:, None], np.arange(N)[None, :], vid] = 1.0
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    qd, kd, vd = to(q[0]), to(k[0]), to(v)
    S = torch.rand((N, D, dv), device="cuda") * 0.01
    z = torch.rand((N, D), device="cuda") + 1.0
    o = torch.empty((steps, N, dv), dtype=torch.bfloat16, device="cuda")
    gd = torch.from_numpy(gen.log_decays(1, steps, N, seed=5001)[0]).cuda()

    def step(t):
        if gated:
            kata.decode_step_decay(qd[t], kd[t], vd[t], gd[t], S, z, out=o[t])
        else:
            kata.decode_step(qd[t], kd[t], vd[t], S, z, out=o[t])

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for t in range(4):
            step(t)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in range(steps):
                step(t)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (reps * steps)
    bytes_step = N * (2 * 4 * D * (dv + 1) + 2 * (2 * dk + 2 * dv) + (4 if gated else 0))
    return ms_step, bytes_step / (ms_step * 1e-3) / 1e9, bytes_step


def decay_gate(kata, torch, gen, steps, warmup):
    """The fwd131k forward with per-token log-decays in [-0.05, 0] against the
    ungated forward on the same inputs (both without state export), for the
    PSD lift and for the first-order feature (orthant inputs); the same for the
    fwd32k (d_k = 32) forward; and the gated decode step."""
    w = gen.WORKLOADS["fwd131k"]
    to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    q, k, v = (to(a) for a in gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype))
    g = torch.from_numpy(gen.log_decays(w.B, w.H, w.T, seed=w.seed + 100)).cuda()
    o = torch.empty_like(v)
    nb = kata.chunked_fwd_decay_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1, "scan")
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ms_g = time_calls(torch, lambda: kata.chunked_fwd_decay_into(q, k, v, g, o, w.chunk, ws),
                      steps, warmup)
    nb2 = kata.chunked_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1, True)
    ws2 = torch.empty(max(nb2, 1), dtype=torch.uint8, device="cuda")
    ms_u = time_calls(torch, lambda: kata.chunked_fwd_into(q, k, v, o, w.chunk, True, ws2),
                      steps, warmup)
    del q, k, v
    q, k, v = (to(a) for a in gen.orthant_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype))
    nb3 = kata.chunked_fwd_decay_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1, "scan",
                                           "identity")
    ws3 = torch.empty(max(nb3, 1), dtype=torch.uint8, device="cuda")
    ms_gi = time_calls(torch, lambda: kata.chunked_fwd_decay_into(
        q, k, v, g, o, w.chunk, ws3, feature="identity"), steps, warmup)
    nb4 = kata.chunked_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1, True, "identity")
    ws4 = torch.empty(max(nb4, 1), dtype=torch.uint8, device="cuda")
    ms_ui = time_calls(torch, lambda: kata.chunked_fwd_into(
        q, k, v, o, w.chunk, True, ws4, feature="identity"), steps, warmup)
    del q, k, v, o, ws, ws2, ws3, ws4
    w32 = gen.WORKLOADS["fwd32k"]
    q, k, v = (to(a) for a in gen.gaussian_qkv(w32.B, w32.H, w32.T, w32.dk, w32.dv, w32.seed,
                                               w32.dtype))
    g = torch.from_numpy(gen.log_decays(w32.B, w32.H, w32.T, seed=w32.seed + 100)).cuda()
    o = torch.empty_like(v)
    nb5 = kata.chunked_fwd_decay_workspace(w32.B, w32.H, w32.T, w32.dk, w32.dv, w32.chunk, 1, "scan")
    ws5 = torch.empty(max(nb5, 1), dtype=torch.uint8, device="cuda")
    ms_g32 = time_calls(torch, lambda: kata.chunked_fwd_decay_into(q, k, v, g, o, w32.chunk, ws5),
                        steps, warmup)
    nb6 = kata.chunked_fwd_workspace(w32.B, w32.H, w32.T, w32.dk, w32.dv, w32.chunk, 1, True)
    ws6 = torch.empty(max(nb6, 1), dtype=torch.uint8, device="cuda")
    ms_u32 = time_calls(torch, lambda: kata.chunked_fwd_into(q, k, v, o, w32.chunk, True, ws6),
                        steps, warmup)
    del q, k, v, o, ws5, ws6
    dms, dgbs, _ = decode_bench(kata, torch, gated=True)
    return {"fwd131k_gated_ms": ms_g, "fwd131k_ungated_ms": ms_u,
            "fwd131k_gated_tokens_per_s": w.B * w.T / (ms_g * 1e-3),
            "gate_overhead": ms_g / ms_u - 1.0,
            "fwd131k_identity_gated_ms": ms_gi, "fwd131k_identity_ungated_ms": ms_ui,
            "identity_gate_overhead": ms_gi / ms_ui - 1.0,
            "fwd32k_gated_ms": ms_g32, "fwd32k_ungated_ms": ms_u32,
            "fwd32k_gate_overhead": ms_g32 / ms_u32 - 1.0,
            "decode_gated_ms_per_step": dms, "decode_gated_GBps": dgbs,
            "decode_gated_hbm_frac": dgbs / PEAK_HBM_GBS}


# A batch-filled shape for the first-order comparison: 256 heads of 4096
# tokens, so that even the sequential walk (one workgroup per head and value
# tile) has 1024 workgroups, four per compute unit.
BATCH4K = dict(name="batch4k", B=16, H=16, T=4096, dk=16, dv=64, chunk=64, seed=12)


def scan_vs_sequential(kata, torch, gen, names, steps, warmup):
    """The inter-chunk prefix by the associative scan (segments in parallel;
    blocked, the default, and the log-depth tree) and by the sequential walk
    (depth N_C: for the PSD lift one workgroup per head, for the first-order
    feature one per head and 16-column value tile), for the PSD lift and for
    the first-order identity feature (orthant inputs), on the same shapes: ms
    per forward, tokens/s, the prefix depth (dependent state combines), the
    workgroups of the output launch and the scan's speedup. The first-order
    feature also runs on a batch-filled shape (BATCH4K) where the sequential
    walk occupies every compute unit, so that its speedup reflects depth
    rather than idle compute units."""
    import types
    out = {}
    speedups, first_order = [], []
    to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    cases = [(gen.WORKLOADS[n], f) for n in names for f in ("psd", "identity")]
    cases.append((types.SimpleNamespace(**BATCH4K), "identity"))
    for w, feature in cases:
        draw = gen.gaussian_qkv if feature == "psd" else gen.orthant_qkv
        q, k, v = (to(a) for a in draw(w.B, w.H, w.T, w.dk, w.dv, w.seed, "bf16"))
        o = torch.empty_like(v)
        row = {}
        for prefix in ("scan", "tree", "sequential"):
            nbytes = kata.chunked_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1, True,
                                                feature, prefix)
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
            n = steps if prefix != "sequential" else max(1, min(steps, 3))
            ms = time_calls(torch, lambda: kata.chunked_fwd_into(
                q, k, v, o, w.chunk, True, ws, feature=feature, prefix=prefix), n,
                min(warmup, 1) if prefix == "sequential" else warmup)
            row[prefix] = {"ms": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
                           "depth": kata.prefix_depth(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1,
                                                      feature, prefix)}
            if prefix == "sequential":
                row[prefix]["workgroups"] = w.B * w.H * (w.dv // 16 if feature == "identity" else 1)
            del ws
        row["scan_speedup"] = row["sequential"]["ms"] / row["scan"]["ms"]
        row["tree_speedup"] = row["sequential"]["ms"] / row["tree"]["ms"]
        speedups.append(row["scan_speedup"])
        if feature == "identity":
            first_order.append(row["scan_speedup"])
        out[f"{w.name}/{feature}"] = row
        del q, k, v, o
    out["geomean_scan_speedup"] = float(np.exp(np.mean(np.log(speedups))))
    out["geomean_first_order_scan_speedup"] = float(np.exp(np.mean(np.log(first_order))))
    return out


def scan_states_bench(kata, torch, gen, names, steps, warmup):
    """kata_scan_states (per-chunk exclusive prefix states: segment states, the
    scan over segment records, then a walk of each segment writing every
    chunk's packed prefix) on the fwd131k and fwd32k shapes: ms per call and
    GB/s over its minimal traffic (k, v read once; every prefix S, z and the
    final state written once)."""
    out = {}
    to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    for name in names:
        w = gen.WORKLOADS[name]
        _, k, v = (to(a) for a in gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, "bf16"))
        D = w.dk * (w.dk + 1) // 2
        NC = -(-w.T // w.chunk)
        BH = w.B * w.H
        Sp = torch.empty((w.B, w.H, NC, D, w.dv), device="cuda")
        zp = torch.empty((w.B, w.H, NC, D), device="cuda")
        ST = torch.empty((w.B, w.H, D, w.dv), device="cuda")
        zT = torch.empty((w.B, w.H, D), device="cuda")
        nws = kata.lib().kata_scan_states_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        ms = time_calls(torch, lambda: kata.scan_states_into(k, v, w.chunk, Sp, zp, ST, zT,
                                                             workspace=ws), steps, warmup)
        nbytes = BH * (w.T * 2 * (w.dk + w.dv) + (NC + 1) * 4 * D * (w.dv + 1))
        scan_bytes = BH * NC * 2 * 4 * D * (w.dv + 1)
        out[name] = {"ms": ms, "alg_bytes": nbytes, "alg_GBps": nbytes / (ms * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "scan_alone_bytes": scan_bytes}
        del k, v, Sp, zp, ST, zT, ws
    return out


def recall_forward(kata, torch, gen, steps, warmup):
    """The recall-shaped stream workload (B=8, H=4, T=16384, d_k=16, d_v=64,
    C=64): keys from per-stream codebooks with overwrites, one-hot values."""
    w = gen.WORKLOADS["recall16k"]
    to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    q, k, v = (to(a) for a in gen.recall_stream(w.B, w.H, w.T, w.dk, w.dv, w.seed))
    ms, wall, phases = time_forward(kata, torch, w, q, k, v, steps, warmup)
    return {"tokens_per_s": w.B * w.T / (ms * 1e-3), "ms_per_step": ms, "phase_ms": phases,
            "hbm_frac_alg_whole_step":
                alg_bytes_per_token_head(w.dk, w.dv) * w.B * w.H * w.T / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def delta_forward(kata, torch, gen, steps, warmup):
    """DeltaKATA (kata_delta_fwd: the per-chunk inverse kernel, then the chunk
    walk) on the recall-shaped stream at full size (B=8, H=4, T=16384, d_k=16,
    d_v=64, C=64) with write strength 1 (the overwrite the delta rule is for):
    ms, tokens/s and its fp32 rate against the fp32 peak (157.3 TFLOP/s, the
    same for the vector ALUs and the fp32 matrix cores the products run on).
    Algorithmic flops per token-head (fp32 FMAs x 2, the whole state of d_v + 1
    columns once): the products K A, phi(Q) A and K^T P over D (3 x 2 D (d_v+1)),
    the lower-triangular T R and masked-weight products (2 x 2 (C/2) (d_v+1)),
    the chunk's key and query Gram terms (2 x 2 C d_k) and the triangular
    inverse (2 C^2 / 3)."""
    w = gen.WORKLOADS["recall16k"]
    to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    q, k, v = (to(a) for a in gen.recall_stream(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype))
    beta = torch.ones((w.B, w.H, w.T), device="cuda")
    o = torch.empty_like(v)
    nws = kata.delta_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.chunk, 1)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ms = time_calls(torch, lambda: kata.delta_fwd_into(q, k, v, beta, o, w.chunk, workspace=ws),
                    steps, warmup)
    D, C, cols = w.dk * (w.dk + 1) // 2, w.chunk, w.dv + 1
    per_token = 3 * 2 * D * cols + 2 * 2 * (C // 2) * cols + 2 * 2 * C * w.dk + 2 * C * C / 3
    flops = w.B * w.H * w.T * per_token
    return {"ms": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3), "alg_tflops": flops / (ms * 1e-3) / 1e12,
            "vs_fp32_peak": flops / (ms * 1e-3) / 1e12 / 157.3,
            "workgroups": w.B * w.H * -(-w.dv // 15), "beta": 1.0, "workload": "recall16k"}


def factored_forward(kata, torch, gen, steps, warmup):
    """KATA-Mg ("multi") and KATA-Sigma-g ("summed") through kata_factored_fwd
    (state export included) on the fwd131k inputs (B=1, H=8, T=131072, d_k=16,
    d_v=64, C=64) with 2 and 4 factors, and on the fwd32k inputs (B=1, H=16,
    T=32768, d_k=32, d_v=64) at C=64: ms, tokens/s and the algorithmic HBM rate
    of the step (q, k, v read once, o written once)."""
    out = {}
    for name, cases in (("fwd131k", ((2, "multi"), (2, "summed"), (4, "multi"), (4, "summed"))),
                        ("fwd32k", ((4, "multi"), (4, "summed"), (2, "summed")))):
        w = gen.WORKLOADS[name]
        to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
        q, k, v = (to(a) for a in gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype))
        o = torch.empty_like(v)
        nbytes = (2 * w.dk + 2 * w.dv) * 2 * w.B * w.H * w.T
        for g, kind in cases:
            D = kata.factored_dim(w.dk, g, kind)
            S = torch.empty((w.B, w.H, D, w.dv), dtype=torch.float32, device="cuda")
            z = torch.empty((w.B, w.H, D), dtype=torch.float32, device="cuda")
            wsb = kata.factored_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, 64, 1, True, g, kind)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
            ms = time_calls(torch, lambda: kata.factored_fwd_into(q, k, v, o, g, kind, 64, True, ws,
                                                                  S_out=S, z_out=z), steps, warmup)
            out[f"{name}/{kind}{g}"] = {
                "ms": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3), "features": D,
                "alg_GBps": nbytes / (ms * 1e-3) / 1e9,
                "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
            del ws, S, z
        del q, k, v, o
    return out


def box_peaks(torch):
    """Measured yardsticks on this GPU: a large bf16 GEMM through torch and a 1 GiB
    device-to-device copy (bytes read + written per second)."""
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms_mm = time_calls(torch, lambda: torch.mm(a, b), 10, 3)
    del a, b
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    ms_cp = time_calls(torch, lambda: y.copy_(x), 10, 3)
    nbytes = 2 * x.numel() * 4
    del x, y
    return {"bf16_gemm_tflops": 2 * n ** 3 / (ms_mm * 1e-3) / 1e12,
            "copy_GBps": nbytes / (ms_cp * 1e-3) / 1e9,
            "gemm": f"torch.mm bf16 {n}x{n}x{n}", "copy": "1 GiB fp32 device-to-device copy_"}


def cpu_chunked(w, q, k, v, budget_s):
    """The float64 chunked-form oracle (O(T) per head) on head (0, 0) of the
    workload, on prefixes of 8192 tokens repeated until the budget is spent;
    tokens/s = token-heads per second / H."""
    import oracle as O
    Tp = min(8192, w.T)
    qq, kk, vv = q[:1, :1, :Tp], k[:1, :1, :Tp], v[:1, :1, :Tp]
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        O.chunked(qq, kk, vv, w.chunk)
        done += Tp
    el = time.perf_counter() - t0
    return {"value": done / (w.H * el), "unit": "tokens/s", "kind": "oracle (chunked form)",
            "sample": f"float64 chunked form, C={w.chunk}, on the first {Tp} tokens of head (0,0) "
                      f"of the {w.name} workload, {done // Tp} passes in {el:.1f} s; "
                      "tokens/s = token-heads/(H*s)"}


def host_description():
    """CPU model (from /proc/cpuinfo), cores available to this process, and the
    BLAS library numpy uses with its thread count."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)
            threads = sum(i.get("num_threads", 0) for i in libs)
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)),
            "blas": blas, "blas_threads": threads}


def cpu_baseline(w, q, k, v, budget_s):
    """The float64 brute-force oracle on a bounded sample of query rows of the
    same workload (head 0, uniformly drawn positions), scaled to tokens/s."""
    import oracle as O
    hostd = host_description()
    cores = hostd["blas_threads"] or hostd["cores_available"]
    rng = np.random.Generator(np.random.PCG64(99))
    qq, kk, vv = q[:1, :1], k[:1, :1], v[:1, :1]
    rows_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        rows = np.sort(rng.integers(0, w.T, 64))
        O.brute_force_rows(qq, kk, vv, rows)
        rows_done += rows.size
    el = time.perf_counter() - t0
    tok_s = rows_done / (w.H * el)     # each token needs H head-rows
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 brute force on {rows_done} uniformly drawn query rows of head "
                      f"(0,0) of the {w.name} workload in {el:.1f} s; tokens/s = rows/(H*s)",
            "cpu_model": hostd["cpu_model"], "blas": hostd["blas"],
            "cores_available": hostd["cores_available"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--quick", action="store_true", help="primary workload only (for profiling)")
    ap.add_argument("--workload", default="fwd131k",
                    help="with --quick: the forward workload to time (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scales HBM counters)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode steps (2048 rows, then 32768 rows; for counter runs)")
    ap.add_argument("--only", choices=["factored", "scan_vs_sequential", "scan_states", "delta",
                                       "quadratic"],
                    help="run one part of parts.* alone and print it (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(see the sharding paragraph of the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4,
                          "launches": 3}), flush=True)
        return
    import kernelized_linear_attention_phi_amd as kata
    from kernelized_linear_attention_phi_amd import inputs as gen
    kata.lib()
    if args.only:
        part = {"factored": lambda: factored_forward(kata, torch, gen, args.steps, args.warmup),
                "scan_vs_sequential": lambda: scan_vs_sequential(
                    kata, torch, gen, ("fwd4k", "fwd32k", "fwd131k"), args.steps, args.warmup),
                "scan_states": lambda: scan_states_bench(kata, torch, gen, ["fwd131k", "fwd32k"],
                                                         args.steps, args.warmup),
                "delta": lambda: delta_forward(kata, torch, gen, 3, 1),
                "quadratic": lambda: quadratic_vs_chunked(kata, torch, gen, "fwd4k", args.steps,
                                                          args.warmup)}[args.only]
        print(json.dumps(part()), flush=True)
        return
    if args.decode_only:
        out = {}
        for n_seq, steps in ((512, 64), (8192, 16)):
            dms, dgbs, dbytes = decode_bench(kata, torch, steps=steps, n_seq=n_seq, reps=1)
            out[f"rows{4 * n_seq}"] = {"ms_per_step": dms, "alg_GBps": dgbs, "bytes_per_step": dbytes,
                                       "steps": steps}
        print(json.dumps(out), flush=True)
        return

    def progress(part):
        print(f"bench: {part} done", file=sys.stderr, flush=True)

    def load(name):
        w = gen.WORKLOADS[name]
        q, k, v = gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype)
        to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
        return w, (q, k, v), (to(q), to(k), to(v))

    if args.workload != "fwd131k" and not args.quick:
        print("--workload only applies with --quick", file=sys.stderr)
        sys.exit(2)
    w, host_in, dev_in = load(args.workload)
    ms, wall_ms, phases = time_forward(kata, torch, w, *dev_in, args.steps, args.warmup)
    progress(w.name)
    tok = w.B * w.T
    value = tok / (ms * 1e-3)
    th = w.B * w.H * w.T
    flops = alg_flops_per_token_head(w.dk, w.dv, w.chunk) * th
    abytes = alg_bytes_per_token_head(w.dk, w.dv) * th
    out_ms = phases["output"]
    achieved = abytes / (out_ms * 1e-3) / 1e9
    cold = None
    if not args.quick:
        # three input/output sets (3 x 335 MB) rotated through the timed steps:
        # each step's inputs were last touched two steps earlier, beyond the
        # 256 MB memory-side cache
        sets = [dev_in + (torch.empty_like(dev_in[2]),)]
        for r in (1, 2):
            qh, kh, vh = gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed + 1000 * r, w.dtype)
            to = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
            sets.append((to(qh), to(kh), to(vh), torch.empty_like(dev_in[2])))
            del qh, kh, vh
        ms_c, _, ph_c = time_forward(kata, torch, w, None, None, None, args.steps, args.warmup,
                                     sets=sets)
        cold = {"value_cold": tok / (ms_c * 1e-3), "ms_per_step": ms_c, "phase_ms": ph_c,
                "output_kernel_GBps": abytes / (ph_c["output"] * 1e-3) / 1e9,
                "definition": "the same forward with 3 input/output sets (335 MB each) rotated "
                              "through the timed steps, so no step's inputs are resident in "
                              "the 256 MB memory-side cache"}
        del sets
        progress("cold inputs")
    traffic = None
    if w.name == "fwd131k" and os.path.exists(COUNTERS_FILE):
        c = json.load(open(COUNTERS_FILE))
        if c.get("kernel_src_sha") == kernel_source_hash():
            traffic = c.get("traffic_bytes_per_launch")
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d_k": w.dk, "d_v": w.dv,
                   "chunk": w.chunk, "causal": True, "state_export": True},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "output phase (fused intra+inter forward)",
                     "alg_bytes_per_launch": abytes, "avg_launch_ms": out_ms},
        "value_cold": None if cold is None else cold["value_cold"],
        "parts": {w.name: {"phase_ms": phases, "wall_ms_per_step": wall_ms,
                              "mfma_util_alg": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                              "alg_tflops": flops / (ms * 1e-3) / 1e12,
                              "hbm_frac_alg_whole_step": abytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}},
    }
    if cold is not None:
        result["parts"][w.name]["cold"] = cold
        result["roofline"]["achieved_cold"] = cold["output_kernel_GBps"]
        result["roofline"]["frac_cold"] = cold["output_kernel_GBps"] / PEAK_HBM_GBS
    if not args.quick:
        del dev_in
        w3, host3, dev3 = load("fwd32k")
        ms3, wall3, ph3 = time_forward(kata, torch, w3, *dev3, args.steps, args.warmup)
        th3 = w3.B * w3.H * w3.T
        fl3 = alg_flops_per_token_head(w3.dk, w3.dv, w3.chunk) * th3
        result["parts"]["fwd32k"] = {
            "tokens_per_s": w3.B * w3.T / (ms3 * 1e-3), "ms_per_step": ms3, "phase_ms": ph3,
            "alg_tflops": fl3 / (ms3 * 1e-3) / 1e12,
            "mfma_util_alg": fl3 / (ms3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "mfma_util_alg_output_phase": fl3 / (ph3["output"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del dev3
        progress("fwd32k")
        result["parts"]["fwd4k"] = quadratic_vs_chunked(kata, torch, gen, "fwd4k", args.steps,
                                                        args.warmup)
        progress("fwd4k")
        result["parts"]["scan_vs_sequential"] = scan_vs_sequential(
            kata, torch, gen, ("fwd4k", "fwd32k", "fwd131k"), min(args.steps, 10), args.warmup)
        progress("scan_vs_sequential")
        result["parts"]["scan_states"] = scan_states_bench(kata, torch, gen, ["fwd131k", "fwd32k"],
                                                           min(args.steps, 10), min(args.warmup, 3))
        progress("scan_states")
        result["parts"]["decay_gate"] = decay_gate(kata, torch, gen, min(args.steps, 10),
                                                   args.warmup)
        progress("decay_gate")
        result["parts"]["recall16k"] = recall_forward(kata, torch, gen, min(args.steps, 10),
                                                      args.warmup)
        result["parts"]["delta_recall16k"] = delta_forward(kata, torch, gen, 3, 1)
        result["parts"]["factored"] = factored_forward(kata, torch, gen, min(args.steps, 10),
                                                       min(args.warmup, 3))
        progress("recall16k and delta")
        dms, dgbs, dbytes = decode_bench(kata, torch)
        result["parts"]["decode"] = {"ms_per_step": dms, "alg_GBps": dgbs,
                                     "hbm_frac": dgbs / PEAK_HBM_GBS, "bytes_per_step": dbytes,
                                     "rows": 2048, "steps": 1024, "hip_graph": True,
                                     "state_MB": 2048 * 4 * 136 * 65 / 1e6,
                                     "note": "state fits the 256 MB memory-side cache: cache-assisted"}
        cold = {}
        for n_seq, steps in ((2048, 128), (8192, 48)):
            dms, dgbs, dbytes = decode_bench(kata, torch, steps=steps, n_seq=n_seq, reps=2)
            rows = 4 * n_seq
            cold[f"rows{rows}"] = {
                "ms_per_step": dms, "alg_GBps": dgbs, "hbm_frac": dgbs / PEAK_HBM_GBS,
                "bytes_per_step": dbytes, "rows": rows, "steps": steps, "hip_graph": True,
                "state_MB": rows * 4 * 136 * 65 / 1e6}
        cold["note"] = ("states of 290 MB and 1.16 GB, beyond the 256 MB memory-side cache "
                        "(the larger one four times over), swept once per step")
        result["parts"]["decode_cold"] = cold
        progress("decode")
        peaks = box_peaks(torch)
        result["parts"]["box_peaks"] = peaks
        result["roofline"]["frac_vs_measured_copy"] = achieved / peaks["copy_GBps"]
        for key, row in result["parts"]["decode_cold"].items():
            if isinstance(row, dict):
                row["frac_vs_measured_copy"] = row["alg_GBps"] / peaks["copy_GBps"]
        result["parts"]["fwd32k"]["mfma_util_vs_measured_gemm"] = (
            result["parts"]["fwd32k"]["alg_tflops"] / peaks["bf16_gemm_tflops"])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, *host_in, args.cpu_budget)
        result["parts"]["cpu_chunked_oracle"] = cpu_chunked(w, *host_in, args.cpu_budget / 2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
