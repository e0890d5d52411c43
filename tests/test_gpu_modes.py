"""GPU parity of the first-order (identity) feature and of the sequential
inter-chunk prefix, both through kata_chunked_fwd_ex, against the float64
oracles (oracle/first_order_oracle.py and the PSD-lift oracle).

bf16 inputs with fp32 accumulation: tolerance 2e-2 (row-normwise), as for the
PSD lift. Identity-feature inputs lie on the nonnegative orthant (unit rows of
|N(0, I)|), where its weights q.k are nonnegative and the output is a convex
combination of values; a zero denominator must give exactly 0.

Final states: 1e-5 for the identity feature (its state products k v of bf16
inputs are exact in fp32, so only fp32 summation order differs) and 2e-2 for
the PSD lift (the lifted key products are rounded to bf16 before the matrix
cores, as in the scan-prefix parity tests)."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, sample_rows, say, state_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
PSD_STATE_TOL = 2e-2


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def run(kata, q, k, v, C, feature, prefix, causal=True, S0=None, z0=None, state=False,
        dtype="bf16"):
    """kata_chunked_fwd_ex with every output and the workspace pre-filled with
    NaN (an element the library fails to write, or scratch it reads before
    writing, cannot pass for a correct value)."""
    import torch
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    B, H, T, dk = qd.shape
    dv = vd.shape[-1]
    D = kata.feature_dim(dk, feature)
    nan = float("nan")
    o = torch.full_like(vd, nan)
    S_out = torch.full((B, H, D, dv), nan, device="cuda") if state else None
    z_out = torch.full((B, H, D), nan, device="cuda") if state else None
    nbytes = kata.chunked_fwd_workspace(B, H, T, dk, dv, C, 1 if dtype == "bf16" else 0, causal,
                                        feature, prefix)
    ws = torch.full((max(nbytes, 4) // 4,), nan, device="cuda")
    kata.chunked_fwd_into(qd, kd, vd, o, C, causal, ws,
                          S0=None if S0 is None else dev(S0), z0=None if z0 is None else dev(z0),
                          S_out=S_out, z_out=z_out, feature=feature, prefix=prefix)
    torch.cuda.synchronize()
    if state:
        return host(o), host(S_out), host(z_out)
    return host(o)


# ---- first-order feature ---------------------------------------------------------

@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("dk,dv", [(16, 64), (16, 16), (16, 32), (32, 64), (32, 16)])
@pytest.mark.parametrize("C", [32, 64, 128])
def test_identity_causal(kata, prefix, dk, dv, C):
    """Several chunks and a ragged tail; every output and the final state."""
    B, H, T = 2, 3, 1000
    q, k, v = gen.orthant_qkv(B, H, T, dk, dv, seed=900 + dk + dv + C, dtype="bf16")
    say(f"identity {prefix} dk={dk} dv={dv} C={C}")
    o, S, z = run(kata, q, k, v, C, "identity", prefix, state=True)
    assert row_rel_err(o, O.fo_brute_force(q, k, v)) <= TOL
    St, zt = O.fo_state_from_tokens(k, v)
    assert state_rel_err(S, St) <= 1e-5 and state_rel_err(z, zt) <= 1e-5


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 200])
def test_identity_lengths(kata, prefix, T):
    q, k, v = gen.orthant_qkv(1, 2, T, 16, 64, seed=950 + T, dtype="bf16")
    say(f"identity {prefix} T={T}")
    o = run(kata, q, k, v, 64, "identity", prefix)
    assert row_rel_err(o, O.fo_brute_force(q, k, v)) <= TOL
    if T == 1:       # a single token: (w v) / w rounds back to v
        assert np.array_equal(o, v.astype(np.float64))


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("dk", [16, 32])
def test_identity_noncausal(kata, prefix, dk):
    q, k, v = gen.orthant_qkv(2, 2, 333, dk, 64, seed=960 + dk, dtype="bf16")
    say(f"identity noncausal {prefix} dk={dk}")
    o, S, z = run(kata, q, k, v, 64, "identity", prefix, causal=False, state=True)
    assert row_rel_err(o, O.fo_brute_force(q, k, v, causal=False)) <= TOL
    St, zt = O.fo_state_from_tokens(k, v)
    assert state_rel_err(S, St) <= 1e-5 and state_rel_err(z, zt) <= 1e-5


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
@pytest.mark.parametrize("dk,C", [(16, 64), (32, 128)])
def test_identity_resume(kata, prefix, dk, C):
    """An initial state standing for earlier tokens: outputs and final state
    equal the oracle over the whole sequence."""
    T1, T2 = 300, 450
    q, k, v = gen.orthant_qkv(1, 3, T1 + T2, dk, 64, seed=970 + dk, dtype="bf16")
    S0, z0 = O.fo_state_from_tokens(k[:, :, :T1], v[:, :, :T1])
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    say(f"identity resume {prefix} dk={dk} C={C}")
    o, S, z = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], C, "identity", prefix,
                  S0=S0, z0=z0, state=True)
    assert row_rel_err(o, O.fo_brute_force(q, k, v)[:, :, T1:]) <= TOL
    St, zt = O.fo_state_from_tokens(k, v)
    assert state_rel_err(S, St) <= 1e-5 and state_rel_err(z, zt) <= 1e-5


@pytest.mark.parametrize("prefix", ["scan", "sequential"])
def test_identity_integer_probe_bit_exact(kata, prefix):
    """Basis keys and queries, small integer values: weights are 0 or 1, states
    are small integers (exact in bf16 below 256) and every output equals the
    exact ratio rounded to bf16."""
    r = np.random.Generator(np.random.PCG64(5))
    T, d, dv = 600, 16, 64
    k = np.eye(d)[r.integers(0, d, (1, 2, T))].astype(np.float32)
    q = np.eye(d)[r.integers(0, d, (1, 2, T))].astype(np.float32)
    v = r.integers(-3, 4, (1, 2, T, dv)).astype(np.float32)
    say(f"identity integer probe {prefix}")
    o, S, z = run(kata, q, k, v, 64, "identity", prefix, state=True)
    want = gen.round_to(O.fo_brute_force(q, k, v), "bf16").astype(np.float64)
    assert np.array_equal(o, want)
    St, zt = O.fo_state_from_tokens(k, v)
    assert np.array_equal(S, St) and np.array_equal(z, zt)


def test_identity_bitwise_causality(kata):
    T = 300
    q, k, v = gen.orthant_qkv(1, 2, T, 16, 64, seed=980, dtype="bf16")
    say("identity causality")
    base = run(kata, q, k, v, 64, "identity", "scan")
    for j in [63, 64, 127, 128, 255]:
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        k2[:, :, j] = gen.round_to(k[:, :, j][..., ::-1] + 0.5, "bf16")
        v2[:, :, j] = gen.round_to(v[:, :, j] * 3.0 + 1.0, "bf16")
        got = run(kata, q2, k2, v2, 64, "identity", "scan")
        assert np.array_equal(got[:, :, :j], base[:, :, :j]), f"output before {j} changed"
        assert not np.array_equal(got[:, :, j], base[:, :, j])


def test_identity_zero_rows(kata):
    q, k, v = gen.orthant_qkv(1, 1, 200, 16, 64, seed=985, dtype="bf16")
    q[:, :, 5] = 0.0
    q[:, :, 150] = 0.0
    o = run(kata, q, k, v, 64, "identity", "scan")
    assert np.all(o[:, :, 5] == 0.0) and np.all(o[:, :, 150] == 0.0)
    assert row_rel_err(o, O.fo_brute_force(q, k, v)) <= TOL


def test_identity_fullsize_fwd4k(kata):
    """The 4k workload's shape on the orthant, every output, both prefixes."""
    w = gen.WORKLOADS["fwd4k"]
    q, k, v = gen.orthant_qkv(w.B, w.H, w.T, w.dk, w.dv, seed=w.seed, dtype="bf16")
    ref = O.fo_brute_force(q, k, v)
    for prefix in ("scan", "sequential"):
        say(f"identity full size fwd4k {prefix}")
        assert row_rel_err(run(kata, q, k, v, w.chunk, "identity", prefix), ref) <= TOL


# ---- sequential prefix, PSD lift ---------------------------------------------------

@pytest.mark.parametrize("dtype,dk,dv,C", [("f32", 16, 64, 64), ("f32", 32, 16, 128),
                                           ("bf16", 16, 64, 16), ("f32", 16, 32, 16)])
def test_identity_valu_path(kata, dtype, dk, dv, C):
    """The first-order feature on the fp32 path (fp32 inputs, or chunk 16):
    causal with a ragged tail and the final state, non-causal, and resume from an
    initial state."""
    B, H, T = 2, 2, 333
    q, k, v = gen.orthant_qkv(B, H, T, dk, dv, seed=1700 + dk + dv + C, dtype=dtype)
    tol = 1e-4 if dtype == "f32" else TOL
    say(f"identity valu dtype={dtype} dk={dk} dv={dv} C={C}")
    o, S, z = run(kata, q, k, v, C, "identity", "scan", state=True, dtype=dtype)
    assert row_rel_err(o, O.fo_brute_force(q, k, v)) <= tol
    St, zt = O.fo_state_from_tokens(k, v)
    assert state_rel_err(S, St) <= 1e-5 and state_rel_err(z, zt) <= 1e-5
    o = run(kata, q, k, v, C, "identity", "scan", causal=False, dtype=dtype)
    assert row_rel_err(o, O.fo_brute_force(q, k, v, causal=False)) <= tol
    T1 = 120
    S0, z0 = O.fo_state_from_tokens(k[:, :, :T1], v[:, :, :T1])
    o = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], C, "identity", "scan",
            S0=S0.astype(np.float32), z0=z0.astype(np.float32), dtype=dtype)
    assert row_rel_err(o, O.fo_brute_force(q, k, v)[:, :, T1:]) <= tol


@pytest.mark.parametrize("dk,dv,C", [(16, 64, 64), (16, 16, 32), (16, 32, 64), (32, 64, 128),
                                     (32, 32, 64), (32, 16, 64)])
def test_psd_sequential(kata, dk, dv, C):
    B, H, T = 2, 3, 1000
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=1000 + dk + dv + C, dtype="bf16")
    say(f"psd sequential dk={dk} dv={dv} C={C}")
    o, S, z = run(kata, q, k, v, C, "psd", "sequential", state=True)
    assert row_rel_err(o, O.brute_force(q, k, v)) <= TOL
    St, zt = O.state_from_tokens(k, v)
    assert state_rel_err(S, St) <= PSD_STATE_TOL and state_rel_err(z, zt) <= PSD_STATE_TOL


@pytest.mark.parametrize("dk,C", [(16, 64), (32, 128)])
def test_psd_sequential_resume_and_noncausal(kata, dk, C):
    T1, T2 = 300, 450
    q, k, v = gen.gaussian_qkv(1, 3, T1 + T2, dk, 64, seed=1050 + dk, dtype="bf16")
    S0, z0 = O.state_from_tokens(k[:, :, :T1], v[:, :, :T1])
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    say(f"psd sequential resume dk={dk}")
    o, S, z = run(kata, q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], C, "psd", "sequential",
                  S0=S0, z0=z0, state=True)
    assert row_rel_err(o, O.brute_force(q, k, v)[:, :, T1:]) <= TOL
    St, zt = O.state_from_tokens(k, v)
    assert state_rel_err(S, St) <= PSD_STATE_TOL and state_rel_err(z, zt) <= PSD_STATE_TOL
    say(f"psd sequential noncausal dk={dk}")
    o = run(kata, q, k, v, C, "psd", "sequential", causal=False)
    assert row_rel_err(o, O.brute_force(q, k, v, causal=False)) <= TOL


def test_psd_sequential_fullsize_fwd4k(kata):
    """The 4k workload at full size: sampled rows against the oracle, and within
    tolerance of the scan-prefix output."""
    from tests.gpu_util import workload_inputs
    w, q, k, v, _ = workload_inputs("fwd4k")
    say("psd sequential full size fwd4k")
    o_seq = run(kata, q, k, v, w.chunk, "psd", "sequential")
    o_scan = run(kata, q, k, v, w.chunk, "psd", "scan")
    rows = sample_rows(w.T, w.chunk)
    ref = O.brute_force_rows(q, k, v, rows)
    assert row_rel_err(o_seq[:, :, rows], ref) <= TOL
    assert row_rel_err(o_seq, o_scan) <= 2 * TOL


def test_modes_deterministic(kata):
    """Repeated calls agree bit for bit (an output row staged in LDS by one
    wavefront and stored by another must not be overwritten before it is read)."""
    for dk in (16, 32):
        q, k, v = gen.orthant_qkv(2, 4, 1500, dk, 64, seed=1100, dtype="bf16")
        for feature in ("identity", "psd"):
            for prefix in ("scan", "sequential"):
                for C in (64, 128) if dk == 32 or feature == "identity" else (32, 64):
                    a = run(kata, q, k, v, C, feature, prefix)
                    for _ in range(3):
                        assert np.array_equal(a, run(kata, q, k, v, C, feature, prefix)), \
                            (dk, feature, prefix, C)
