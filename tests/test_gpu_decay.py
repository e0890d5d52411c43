"""GPU parity of the decay-gated forward (kata_chunked_fwd_decay) and decode step
(kata_decode_step_decay) against the float64 decay oracle
(oracle/decay_oracle.py).

Matrix-core paths (bf16; PSD lift at d_k = 16 with C in {32, 64} and at
d_k = 32 with C in {64, 128}; first-order feature with C in {32, 64}; T a
multiple of 4 across heads): fp32 accumulation, outputs within 2e-2
(row-normwise). The gated PSD kernels take split (hi + lo) bf16 operands for
every lifted feature, state entry and Gram product, so their final states are
fp32-accurate sums (within 1e-4 of the state norm) and strong gates, which
leave only a few keys in the state, still meet 2e-2. The first-order kernels
round scaled keys to bf16 (states within 2e-2). VALU path (every other shape): fp32 arithmetic
throughout, outputs within 1e-4 for fp32 inputs and 2e-2 for bf16 (the bf16
rounding of the output), states within 1e-4. The decode step is fp32
arithmetic on the state (1e-5 for fp32 inputs)."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, sample_rows, say, state_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
STATE_TOL = 2e-2          # first-order matrix-core kernels (bf16 keys after scaling)
PSD_STATE_TOL = 1e-4      # gated PSD kernels: split operands, fp32-accurate sums


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def run(kata, q, k, v, g, C, prefix, S0=None, z0=None, state=False, dtype="bf16", feature="psd",
        G=0):
    """kata_chunked_fwd_decay with outputs and workspace pre-filled with NaN."""
    import torch
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    gd = dev(g)
    B, H, T, dk = qd.shape
    dv = vd.shape[-1]
    D = kata.feature_dim(dk, feature)
    nan = float("nan")
    o = torch.full_like(vd, nan)
    S_out = torch.full((B, H, D, dv), nan, device="cuda") if state else None
    z_out = torch.full((B, H, D), nan, device="cuda") if state else None
    nbytes = kata.chunked_fwd_decay_workspace(B, H, T, dk, dv, C, 1 if dtype == "bf16" else 0,
                                              prefix, feature, segment_chunks=G)
    ws = torch.full((max(nbytes, 4) // 4,), nan, device="cuda")
    kata.chunked_fwd_decay_into(qd, kd, vd, gd, o, C, ws,
                                S0=None if S0 is None else dev(S0), z0=None if z0 is None else dev(z0),
                                S_out=S_out, z_out=z_out, prefix=prefix, feature=feature,
                                segment_chunks=G)
    torch.cuda.synchronize()
    if state:
        return host(o), host(S_out), host(z_out)
    return host(o)


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("dv", [64, 16, 32])
@pytest.mark.parametrize("C", [32, 64])
@pytest.mark.parametrize("gmin", [-0.05, -0.2])
def test_decay_fwd(kata, prefix, dv, C, gmin):
    """Several chunks and a ragged tail; every output and the final state."""
    B, H, T = 2, 3, 1000
    q, k, v = gen.gaussian_qkv(B, H, T, 16, dv, seed=1200 + dv + C, dtype="bf16")
    g = gen.log_decays(B, H, T, seed=1300 + dv + C, gmin=gmin)
    say(f"decay {prefix} dv={dv} C={C} gmin={gmin}")
    o, S, z = run(kata, q, k, v, g, C, prefix, state=True)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("C", [32, 64])
@pytest.mark.parametrize("gmin", [-0.5, -1.0])
def test_decay_strong_gate(kata, prefix, C, gmin):
    """Per-token decays down to exp(-0.5) and exp(-1): the state holds a few
    recent keys. The inter-chunk term evaluates (q.k)^2 through lifted features
    (sum_p phi(q)_p phi(k)_p, terms of size up to |q|^2 |k|^2); with bf16
    operands their rounding would not average out over so few keys (2.3e-2 was
    seen), so the gated kernels split every operand into hi + lo. Every row
    within 2e-2, states within 1e-4."""
    B, H, T = 2, 3, 1000
    q, k, v = gen.gaussian_qkv(B, H, T, 16, 64, seed=1296, dtype="bf16")
    g = gen.log_decays(B, H, T, seed=1396, gmin=gmin)
    say(f"decay strong gate {prefix} C={C} gmin={gmin}")
    o, S, z = run(kata, q, k, v, g, C, prefix, state=True)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
def test_decay_zero_gate_is_ungated(kata, prefix):
    """g = 0: the gated kernels (split operands) give the ungated result, within
    2e-2 of the ungated oracle, and a final state within 1e-4 of the ungated
    one (the bitwise comparison holds on the first-order and fp32 paths; here
    the gated kernels are the more precise of the two)."""
    q, k, v = gen.gaussian_qkv(2, 2, 700, 16, 64, seed=1400, dtype="bf16")
    g = np.zeros((2, 2, 700), np.float32)
    say(f"decay zero gate {prefix}")
    o, S, z = run(kata, q, k, v, g, 64, prefix, state=True)
    assert row_rel_err(o, O.brute_force(q, k, v)) <= TOL
    S_ref, z_ref = O.state_from_tokens(k, v)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


def test_decay_reset(kata):
    """A gate of exp(-1e4) = 0 wipes the state: with no decay after it, later
    outputs equal the ungated oracle on the suffix."""
    q, k, v = gen.gaussian_qkv(1, 2, 600, 16, 64, seed=1410, dtype="bf16")
    g = gen.log_decays(1, 2, 600, seed=1411, gmin=-0.2)
    s = 300
    g[:, :, s] = -1e4
    g[:, :, s + 1:] = 0.0
    say("decay reset")
    for prefix in ("scan", "sequential"):
        o = run(kata, q, k, v, g, 64, prefix)
        assert row_rel_err(o[:, :, s:], O.brute_force(q[:, :, s:], k[:, :, s:], v[:, :, s:])) <= TOL
        assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
def test_decay_resume(kata, prefix):
    """An initial state standing for earlier tokens decays with the sequence."""
    T1, T2 = 300, 452
    q, k, v = gen.gaussian_qkv(1, 3, T1 + T2, 16, 64, seed=1420, dtype="bf16")
    g = gen.log_decays(1, 3, T1 + T2, seed=1421, gmin=-0.05)
    _, S0, z0 = O.decay_recurrent(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1])
    say(f"decay resume {prefix}")
    o, S, z = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:], 64, prefix,
                  S0=S0.astype(np.float32), z0=z0.astype(np.float32), state=True)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)[:, :, T1:]) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 1001])
def test_decay_lengths_single_head(kata, T):
    """One head: any T (the per-head alignment rule only matters across heads)."""
    q, k, v = gen.gaussian_qkv(1, 1, T, 16, 64, seed=1430 + T, dtype="bf16")
    g = gen.log_decays(1, 1, T, seed=1431 + T, gmin=-0.1)
    say(f"decay T={T}")
    o = run(kata, q, k, v, g, 64, "scan")
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL


def test_decay_bitwise_causality(kata):
    q, k, v = gen.gaussian_qkv(1, 2, 300, 16, 64, seed=1440, dtype="bf16")
    g = gen.log_decays(1, 2, 300, seed=1441, gmin=-0.1)
    say("decay causality")
    base = run(kata, q, k, v, g, 64, "scan")
    for j in [63, 64, 127, 128, 255]:
        k2, v2, g2 = k.copy(), v.copy(), g.copy()
        k2[:, :, j] = gen.round_to(k[:, :, j][..., ::-1] + 0.5, "bf16")
        v2[:, :, j] = gen.round_to(v[:, :, j] * 3.0 + 1.0, "bf16")
        g2[:, :, j] = -0.7
        got = run(kata, q, k2, v2, g2, 64, "scan")
        assert np.array_equal(got[:, :, :j], base[:, :, :j]), f"output before {j} changed"
        assert not np.array_equal(got[:, :, j], base[:, :, j])


def test_decay_fullsize_fwd131k(kata):
    """The 131k workload with mild gates: sampled rows against the oracle."""
    from tests.gpu_util import workload_inputs
    w, q, k, v, _ = workload_inputs("fwd131k")
    g = gen.log_decays(w.B, w.H, w.T, seed=1450, gmin=-0.01)
    say("decay full size fwd131k")
    o = run(kata, q, k, v, g, w.chunk, "scan")
    assert np.all(np.isfinite(o))
    rows = sample_rows(w.T, w.chunk, n_random=12)
    assert row_rel_err(o[:, :, rows], O.decay_brute_force_rows(q, k, v, g, rows)) <= TOL


# ---- d_k = 32 on the matrix cores (bf16, chunk 64 or 128) ----------------------------

@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("dv,C", [(64, 128), (16, 128), (32, 64), (64, 64)])
@pytest.mark.parametrize("gmin", [-0.05, -0.2])
def test_decay_fwd32(kata, prefix, dv, C, gmin):
    """d_k = 32: several chunks and segments, a ragged tail; every output and
    the final state."""
    B, H, T = 2, 2, 1000
    q, k, v = gen.gaussian_qkv(B, H, T, 32, dv, seed=1900 + dv + C, dtype="bf16")
    g = gen.log_decays(B, H, T, seed=1901 + C, gmin=gmin)
    say(f"decay d32 {prefix} dv={dv} C={C} gmin={gmin}")
    o, S, z = run(kata, q, k, v, g, C, prefix, state=True)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


@pytest.mark.parametrize("G", [2, 3])
@pytest.mark.parametrize("C", [64, 128])
def test_decay_fwd32_segments(kata, G, C):
    """Segments of several chunks: the output kernel carries the decaying state
    across chunks and the scan combines segment totals with their decays."""
    B, H, T = 1, 3, 1100
    q, k, v = gen.gaussian_qkv(B, H, T, 32, 64, seed=1910 + G + C, dtype="bf16")
    g = gen.log_decays(B, H, T, seed=1911 + G, gmin=-0.05)
    say(f"decay d32 segments G={G} C={C}")
    o, S, z = run(kata, q, k, v, g, C, "scan", state=True, G=G)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("C", [64, 128])
@pytest.mark.parametrize("gmin", [-0.5, -1.0])
def test_decay_fwd32_strong_gate(kata, prefix, C, gmin):
    """Decays down to exp(-0.5) and exp(-1) per token at d_k = 32 (few
    effective keys; split operands as at d_k = 16): every row within 2e-2,
    states within 1e-4."""
    q, k, v = gen.gaussian_qkv(2, 2, 1000, 32, 64, seed=1920, dtype="bf16")
    g = gen.log_decays(2, 2, 1000, seed=1921, gmin=gmin)
    say(f"decay d32 strong gate {prefix} C={C} gmin={gmin}")
    o, S, z = run(kata, q, k, v, g, C, prefix, state=True)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("C", [64, 128])
def test_decay_fwd32_zero_gate_is_ungated(kata, prefix, C):
    """g = 0 at d_k = 32: the ungated result (oracle, 2e-2) and state (1e-4)."""
    q, k, v = gen.gaussian_qkv(2, 2, 700, 32, 64, seed=1930, dtype="bf16")
    g = np.zeros((2, 2, 700), np.float32)
    say(f"decay d32 zero gate {prefix} C={C}")
    o, S, z = run(kata, q, k, v, g, C, prefix, state=True)
    assert row_rel_err(o, O.brute_force(q, k, v)) <= TOL
    S_ref, z_ref = O.state_from_tokens(k, v)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


def test_decay_fwd32_reset(kata):
    """A reset gate inside a chunk at d_k = 32: later outputs equal the ungated
    oracle on the suffix."""
    q, k, v = gen.gaussian_qkv(1, 2, 640, 32, 64, seed=1940, dtype="bf16")
    g = gen.log_decays(1, 2, 640, seed=1941, gmin=-0.2)
    s = 330
    g[:, :, s] = -1e4
    g[:, :, s + 1:] = 0.0
    say("decay d32 reset")
    for prefix in ("scan", "sequential"):
        o = run(kata, q, k, v, g, 128, prefix)
        assert row_rel_err(o[:, :, s:], O.brute_force(q[:, :, s:], k[:, :, s:], v[:, :, s:])) <= TOL
        assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
def test_decay_fwd32_resume(kata, prefix):
    """d_k = 32: an initial state standing for earlier tokens decays with the
    sequence; outputs and the final state."""
    T1, T2 = 300, 452
    q, k, v = gen.gaussian_qkv(1, 3, T1 + T2, 32, 32, seed=1950, dtype="bf16")
    g = gen.log_decays(1, 3, T1 + T2, seed=1951, gmin=-0.05)
    _, S0, z0 = O.decay_recurrent(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1])
    say(f"decay d32 resume {prefix}")
    o, S, z = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:], 128, prefix,
                  S0=S0.astype(np.float32), z0=z0.astype(np.float32), state=True)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)[:, :, T1:]) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= PSD_STATE_TOL and state_rel_err(z, z_ref) <= PSD_STATE_TOL


def test_decay_fwd32_bitwise_causality(kata):
    q, k, v = gen.gaussian_qkv(1, 2, 400, 32, 64, seed=1960, dtype="bf16")
    g = gen.log_decays(1, 2, 400, seed=1961, gmin=-0.1)
    say("decay d32 causality")
    base = run(kata, q, k, v, g, 128, "scan")
    for j in [63, 127, 128, 255, 300]:
        k2, v2, g2 = k.copy(), v.copy(), g.copy()
        k2[:, :, j] = gen.round_to(k[:, :, j][..., ::-1] + 0.5, "bf16")
        v2[:, :, j] = gen.round_to(v[:, :, j] * 3.0 + 1.0, "bf16")
        g2[:, :, j] = -0.7
        got = run(kata, q, k2, v2, g2, 128, "scan")
        assert np.array_equal(got[:, :, :j], base[:, :, :j]), f"output before {j} changed"
        assert not np.array_equal(got[:, :, j], base[:, :, j])


def test_decay_fullsize_fwd32k(kata):
    """The 32k d_k = 32 workload with mild gates: sampled rows against the oracle."""
    from tests.gpu_util import workload_inputs
    w, q, k, v, _ = workload_inputs("fwd32k")
    g = gen.log_decays(w.B, w.H, w.T, seed=1970, gmin=-0.01)
    say("decay full size fwd32k")
    o = run(kata, q, k, v, g, w.chunk, "scan")
    assert np.all(np.isfinite(o))
    rows = sample_rows(w.T, w.chunk, n_random=12)
    assert row_rel_err(o[:, :, rows], O.decay_brute_force_rows(q, k, v, g, rows)) <= TOL


VALU_TOL = {"f32": 1e-4, "bf16": TOL}
VALU_STATE_TOL = 1e-4


@pytest.mark.parametrize("dtype,dk,dv,C", [("f32", 16, 64, 64), ("f32", 32, 16, 32),
                                           ("bf16", 32, 64, 128), ("bf16", 32, 32, 64),
                                           ("bf16", 16, 64, 128), ("bf16", 16, 16, 16),
                                           ("f32", 16, 32, 128)])
@pytest.mark.parametrize("gmin", [-0.05, -0.5])
def test_decay_valu_path(kata, dtype, dk, dv, C, gmin):
    """The fp32 path: shapes without a matrix-core path, and matrix-core
    shapes whose T is not a multiple of 4 across heads (T = 333 here); several
    chunks, a ragged tail, every output and the final state."""
    B, H, T = 2, 2, 333
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=1500 + dk + dv + C, dtype=dtype)
    g = gen.log_decays(B, H, T, seed=1501 + C, gmin=gmin)
    say(f"decay valu dtype={dtype} dk={dk} dv={dv} C={C} gmin={gmin}")
    o, S, z = run(kata, q, k, v, g, C, "scan", state=True, dtype=dtype)
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g)) <= VALU_TOL[dtype]
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= VALU_STATE_TOL and state_rel_err(z, z_ref) <= VALU_STATE_TOL


def test_decay_valu_resume_and_reset(kata):
    """fp32, d_k = 32: an initial state that decays with the sequence, and a
    reset gate (exp(-1e4) = 0) inside a chunk after which the outputs equal the
    ungated oracle on the suffix."""
    T1, T2 = 100, 200
    q, k, v = gen.gaussian_qkv(1, 2, T1 + T2, 32, 64, seed=1510, dtype="f32")
    g = gen.log_decays(1, 2, T1 + T2, seed=1511, gmin=-0.1)
    r = T1 + 70
    g[:, :, r] = -1e4
    g[:, :, r + 1:] = 0.0
    _, S0, z0 = O.decay_recurrent(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1])
    say("decay valu resume and reset")
    o, S, z = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:], 64, "scan",
                  S0=S0.astype(np.float32), z0=z0.astype(np.float32), state=True, dtype="f32")
    full = O.decay_brute_force(q, k, v, g)
    assert row_rel_err(o, full[:, :, T1:]) <= 1e-4
    assert row_rel_err(o[:, :, r - T1:], O.brute_force(q[:, :, r:], k[:, :, r:], v[:, :, r:])) <= 1e-4
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    assert state_rel_err(S, S_ref) <= VALU_STATE_TOL and state_rel_err(z, z_ref) <= VALU_STATE_TOL


def test_decay_valu_zero_gate_matches_ungated(kata):
    """g = 0 on the VALU path gives the ungated VALU forward within rounding."""
    import torch
    q, k, v = gen.gaussian_qkv(1, 2, 300, 32, 64, seed=1520, dtype="f32")
    g = np.zeros((1, 2, 300), np.float32)
    say("decay valu zero gate")
    o = run(kata, q, k, v, g, 128, "scan", dtype="f32")
    ref = host(kata.chunked_fwd(dev(q, "f32"), dev(k, "f32"), dev(v, "f32"), chunk=128))
    torch.cuda.synchronize()
    assert row_rel_err(o, ref) <= 1e-6


def _identity_on_matrix_cores(dtype, C):
    return dtype == "bf16" and C in (32, 64)


@pytest.mark.parametrize("dtype,dk,dv,C", [("f32", 16, 64, 64), ("bf16", 32, 32, 128),
                                           ("bf16", 16, 64, 32), ("f32", 32, 16, 16),
                                           ("bf16", 32, 64, 64), ("bf16", 16, 16, 64)])
@pytest.mark.parametrize("gmin", [-0.05, -0.5])
def test_decay_identity(kata, dtype, dk, dv, C, gmin):
    """The gate on the first-order feature, orthant inputs: every output and the
    final state against the identity-feature decay oracle (matrix cores for bf16
    with chunk 32 or 64, whose keys are rounded to bf16 after scaling: states
    within 2e-2 there, 1e-4 on the VALU path)."""
    B, H, T = 2, 2, 332
    q, k, v = gen.orthant_qkv(B, H, T, dk, dv, seed=1800 + dk + dv + C, dtype=dtype)
    g = gen.log_decays(B, H, T, seed=1801 + C, gmin=gmin)
    say(f"decay identity dtype={dtype} dk={dk} dv={dv} C={C} gmin={gmin}")
    o, S, z = run(kata, q, k, v, g, C, "scan", state=True, dtype=dtype, feature="identity")
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g, feature="identity")) <= VALU_TOL[dtype]
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g, feature="identity")
    stol = STATE_TOL if _identity_on_matrix_cores(dtype, C) else VALU_STATE_TOL
    assert state_rel_err(S, S_ref) <= stol and state_rel_err(z, z_ref) <= stol


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("dk,dv,C", [(16, 64, 64), (32, 16, 32)])
def test_decay_identity_matrix_cores(kata, prefix, dk, dv, C):
    """bf16 first-order gate on the matrix cores with either prefix, a ragged
    tail and an initial state that decays with the sequence."""
    B, H, T1, T2 = 2, 2, 200, 436
    q, k, v = gen.orthant_qkv(B, H, T1 + T2, dk, dv, seed=1830 + dk + C, dtype="bf16")
    g = gen.log_decays(B, H, T1 + T2, seed=1831, gmin=-0.1)
    _, S0, z0 = O.decay_recurrent(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1],
                                  feature="identity")
    say(f"decay identity matrix cores {prefix} dk={dk} dv={dv} C={C}")
    o, S, z = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:], C, prefix,
                  S0=S0.astype(np.float32), z0=z0.astype(np.float32), state=True, feature="identity")
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g, feature="identity")[:, :, T1:]) <= TOL
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g, feature="identity")
    assert state_rel_err(S, S_ref) <= STATE_TOL and state_rel_err(z, z_ref) <= STATE_TOL


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
def test_decay_identity_zero_gate_is_ungated(kata, prefix):
    """g = 0 multiplies by exactly 1: the gated first-order kernels reproduce the
    ungated first-order forward bit for bit."""
    import torch
    q, k, v = gen.orthant_qkv(2, 2, 700, 16, 64, seed=1840, dtype="bf16")
    g = np.zeros((2, 2, 700), np.float32)
    say(f"decay identity zero gate {prefix}")
    o = run(kata, q, k, v, g, 64, prefix, feature="identity")
    ref = host(kata.chunked_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), chunk=64,
                                prefix=prefix, feature="identity"))
    torch.cuda.synchronize()
    assert np.array_equal(o, ref)


def test_decay_identity_reset_and_resume(kata):
    """fp32 first-order feature: an initial state that decays with the sequence
    and a reset gate after which outputs equal the ungated first-order oracle."""
    T1, T2 = 90, 210
    q, k, v = gen.orthant_qkv(1, 2, T1 + T2, 16, 64, seed=1810, dtype="f32")
    g = gen.log_decays(1, 2, T1 + T2, seed=1811, gmin=-0.1)
    r = T1 + 100
    g[:, :, r] = -1e4
    g[:, :, r + 1:] = 0.0
    _, S0, z0 = O.decay_recurrent(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1],
                                  feature="identity")
    say("decay identity resume and reset")
    o = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:], 64, "scan",
            S0=S0.astype(np.float32), z0=z0.astype(np.float32), dtype="f32", feature="identity")
    assert row_rel_err(o, O.decay_brute_force(q, k, v, g, feature="identity")[:, :, T1:]) <= 1e-4
    assert row_rel_err(o[:, :, r - T1:], O.fo_brute_force(q[:, :, r:], k[:, :, r:], v[:, :, r:])) <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk", [16, 32])
def test_decode_decay_chain(kata, dtype, dk):
    """Decode steps with gates from a nonzero state equal the oracle chain."""
    import torch
    N, dv, steps = 64, 64, 5
    q, k, v = gen.gaussian_qkv(1, N, steps, dk, dv, seed=1460 + dk, dtype=dtype)
    g = gen.log_decays(1, N, steps, seed=1461, gmin=-0.3)
    kp, vp = gen.gaussian_qkv(1, N, 20, dk, dv, seed=1462, dtype="f32")[1:]
    S_ref, z_ref = O.state_from_tokens(kp, vp)
    S_ref, z_ref = S_ref[0], z_ref[0]
    S, z = dev(S_ref), dev(z_ref)
    say(f"decode decay dtype={dtype} dk={dk}")
    for t in range(steps):
        o = kata.decode_step_decay(dev(q[0, :, t], dtype), dev(k[0, :, t], dtype),
                                   dev(v[0, :, t], dtype), dev(g[0, :, t]), S, z)
        torch.cuda.synchronize()
        o_ref, S_ref, z_ref = O.decay_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], g[0, :, t],
                                                  S_ref, z_ref)
        assert row_rel_err(host(o), o_ref) <= (1e-5 if dtype == "f32" else TOL)
    assert state_rel_err(host(S), S_ref, lead=1) <= 1e-5
    assert state_rel_err(host(z), z_ref, lead=1) <= 1e-5
