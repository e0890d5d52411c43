"""GPU parity of DeltaKATA (kata_delta_fwd, kata_decode_step_delta) against the
float64 delta oracle (oracle/delta_oracle.py).

The kernels are fp32 throughout. The delta rule's erase can make a readout's
denominator phi(q).z small (about one row in 200 falls below 0.05 with random
unit keys and beta in [0, 1]), and a row's output then carries the absolute
error of its numerator and denominator divided by that denominator. The bar per
row: |o - o_ref|_inf <= tol |o_ref|_inf + 1e-5 (1 + |o_ref|_inf) / |den_ref|,
with tol = 1e-4 for fp32 inputs and 2^-8 for bf16 outputs (their own rounding);
every row whose denominator is at least 0.05 must also meet the plain bar
(1e-4, 2e-2). Final states within 1e-4 of the state norm."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, say, state_rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2.0 ** -8}
PLAIN = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def _betas(B, H, T, seed, lo=0.0, hi=1.0):
    r = np.random.Generator(np.random.PCG64(seed))
    return r.uniform(lo, hi, (B, H, T)).astype(np.float32).astype(np.float64)


def _check_rows(o, num, den, dtype):
    ref = np.where(den[..., None] != 0, num / np.where(den == 0, 1, den)[..., None], 0.0)
    err = np.abs(o - ref).max(-1)
    scale = np.abs(ref).max(-1)
    bound = TOL[dtype] * scale + 1e-5 * (1.0 + scale) / np.maximum(np.abs(den), 1e-30)
    assert np.all(err <= bound), float((err / bound).max())
    ok = np.abs(den) >= 0.05
    assert row_rel_err(o[ok], ref[ok]) <= PLAIN[dtype]
    return ref


def _run(kata, q, k, v, beta, C, dtype, S0=None, z0=None):
    import torch
    init = None if S0 is None else (dev(S0.astype(np.float32)), dev(z0.astype(np.float32)))
    o, (S, z) = kata.delta_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(beta), chunk=C,
                               initial_state=init, return_state=True)
    torch.cuda.synchronize()
    return host(o), host(S), host(z)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,C", [(16, 16, 16), (16, 64, 64), (32, 64, 32), (32, 16, 64),
                                     (16, 32, 32), (32, 32, 16)])
@pytest.mark.parametrize("S0", [False, True])
def test_delta_fwd(kata, dtype, dk, dv, C, S0):
    """Several chunks and a ragged tail, random beta in [0, 1], with and without
    an initial state: every output and the final state."""
    B, H, T = 2, 2, 333
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=6100 + dk + dv + C, dtype=dtype)
    beta = _betas(B, H, T, 6101 + C)
    S0h = z0h = None
    if S0:
        S0h, z0h = O.state_from_tokens(*gen.gaussian_qkv(B, H, 7, dk, dv, seed=6102, dtype="f32")[1:])
    say(f"delta fwd {dtype} dk={dk} dv={dv} C={C} S0={S0}")
    o, S, z = _run(kata, q, k, v, beta, C, dtype, S0h, z0h)
    num, den, S_ref, z_ref = O.delta_recurrent(q, k, v, beta, S0h, z0h, parts=True)
    _check_rows(o, num, den, dtype)
    assert state_rel_err(S, S_ref) <= 1e-4 and state_rel_err(z, z_ref) <= 1e-4


@pytest.mark.parametrize("dk", [16, 32])
def test_delta_chunk_invariance(kata, dk):
    """Chunks of 16, 32 and 64 give the same outputs up to fp32 rounding."""
    q, k, v = gen.gaussian_qkv(1, 3, 500, dk, 64, seed=6200 + dk, dtype="f32")
    beta = _betas(1, 3, 500, 6201)
    say(f"delta chunk invariance dk={dk}")
    outs = [_run(kata, q, k, v, beta, C, "f32") for C in (16, 32, 64)]
    num, den, _, _ = O.delta_recurrent(q, k, v, beta, parts=True)
    for o, S, z in outs:
        _check_rows(o, num, den, "f32")
    for o, S, z in outs[1:]:
        assert state_rel_err(S, outs[0][1]) <= 1e-5


def test_delta_basis_overwrite_exact(kata):
    """Basis-vector keys and queries, integer values, beta = 1: every output is
    exactly the value last written to the queried key (fp32, bit-exact)."""
    r = np.random.Generator(np.random.PCG64(6300))
    B, H, T, d, dv = 1, 2, 300, 16, 16
    ids = r.integers(0, d, (B, H, T))
    k = np.eye(d)[ids]
    v = r.integers(-4, 5, (B, H, T, dv)).astype(np.float64)
    qi = ids.copy()
    for t in range(T):
        qi[:, :, t] = ids[:, :, r.integers(0, t + 1)]
    q = np.eye(d)[qi]
    beta = np.ones((B, H, T))
    say("delta basis overwrite")
    o, _, _ = _run(kata, q, k, v, beta, 64, "f32")
    want = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                last = max(j for j in range(t + 1) if ids[b, h, j] == qi[b, h, t])
                want[b, h, t] = v[b, h, last]
    assert np.array_equal(o, want)


def test_delta_beta_zero(kata):
    """beta = 0 writes nothing: every output reads the initial state and the
    final state equals it bit for bit."""
    q, k, v = gen.gaussian_qkv(1, 2, 200, 16, 64, seed=6400, dtype="f32")
    S0, z0 = O.state_from_tokens(*gen.gaussian_qkv(1, 2, 9, 16, 64, seed=6401, dtype="f32")[1:])
    S0, z0 = S0.astype(np.float32).astype(np.float64), z0.astype(np.float32).astype(np.float64)
    say("delta beta zero")
    o, S, z = _run(kata, q, k, v, np.zeros((1, 2, 200)), 32, "f32", S0, z0)
    fq = O.phi(q)
    assert row_rel_err(o, (fq @ S0) / (fq @ z0[..., None])) <= 1e-5
    assert np.array_equal(S, S0) and np.array_equal(z, z0)


def test_delta_recall_stream(kata):
    """The recall-shaped stream (codebook keys, a quarter of the positions
    re-binding an earlier key, one-hot values) with beta = 1: the delta rule's
    overwrite, against the oracle."""
    q, k, v = gen.recall_stream(2, 2, 2000, 16, 64, seed=6500, dtype="bf16")
    beta = np.ones((2, 2, 2000))
    say("delta recall stream")
    o, S, z = _run(kata, q, k, v, beta, 64, "bf16")
    num, den, S_ref, z_ref = O.delta_recurrent(q, k, v, beta, parts=True)
    _check_rows(o, num, den, "bf16")
    assert state_rel_err(S, S_ref) <= 1e-4 and state_rel_err(z, z_ref) <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 64), (32, 16), (16, 32)])
def test_delta_decode(kata, dtype, dk, dv):
    """Decode steps from a forward's final state: each step and the state
    against the oracle's step (fp32 state, 1e-5)."""
    import torch
    N, T0, steps = 40, 100, 4
    q, k, v = gen.gaussian_qkv(1, N, T0 + steps, dk, dv, seed=6600 + dk + dv, dtype=dtype)
    beta = _betas(1, N, T0 + steps, 6601)
    say(f"delta decode {dtype} dk={dk} dv={dv}")
    _, S, z = _run(kata, q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], beta[:, :, :T0], 32, dtype)
    Sd, zd = dev(S[0]), dev(z[0])
    S_ref, z_ref = S[0], z[0]
    for t in range(T0, T0 + steps):
        od = kata.decode_step_delta(dev(q[0, :, t], dtype), dev(k[0, :, t], dtype),
                                    dev(v[0, :, t], dtype), dev(beta[0, :, t]), Sd, zd)
        torch.cuda.synchronize()
        o_ref, S_ref, z_ref = O.delta_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], beta[0, :, t],
                                                  S_ref, z_ref)
        assert row_rel_err(host(od), o_ref) <= (1e-5 if dtype == "f32" else 2e-2)
        S_ref, z_ref = host(Sd), host(zd)          # next step from the GPU's state
    _, S_all, z_all = O.delta_recurrent(q, k, v, beta)
    assert state_rel_err(host(Sd), S_all[0], lead=1) <= 1e-4
    assert state_rel_err(host(zd), z_all[0], lead=1) <= 1e-4


def test_delta_fullsize_recall16k(kata):
    """The recall-shaped workload at full size (B=8, H=4, T=16384, beta = 1),
    every output and the final state against the oracle's recurrence."""
    w = gen.WORKLOADS["recall16k"]
    q, k, v = gen.recall_stream(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype)
    beta = np.ones((w.B, w.H, w.T))
    say("delta fullsize recall16k")
    o, S, z = _run(kata, q, k, v, beta, 64, "bf16")
    num, den, S_ref, z_ref = O.delta_recurrent(q, k, v, beta, parts=True)
    _check_rows(o, num, den, "bf16")
    assert state_rel_err(S, S_ref) <= 1e-4 and state_rel_err(z, z_ref) <= 1e-4


@pytest.mark.parametrize("dk,C", [(16, 64), (32, 16)])
@pytest.mark.parametrize("T", [1, 5, 17, 64, 65])
def test_delta_short_sequences(kata, dk, C, T):
    """Sequences of one token, shorter than a chunk, exactly one chunk and one
    past it, over 15 heads (not a multiple of 8, so some workgroups of the chunk
    walk fall past the last head): outputs and final state."""
    B, H, dv = 3, 5, 32
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=6700 + T + dk, dtype="bf16")
    beta = _betas(B, H, T, 6701 + T)
    say(f"delta short dk={dk} C={C} T={T}")
    o, S, z = _run(kata, q, k, v, beta, C, "bf16")
    num, den, S_ref, z_ref = O.delta_recurrent(q, k, v, beta, parts=True)
    _check_rows(o, num, den, "bf16")
    assert state_rel_err(S, S_ref) <= 1e-4 and state_rel_err(z, z_ref) <= 1e-4


def test_delta_caller_workspace_reused(kata):
    """A caller-owned workspace sized for a long call serves a shorter call
    next; both equal the calls that allocate their own (bit for bit)."""
    import torch
    B, H, dk, dv, C = 1, 3, 16, 64, 64
    nws = kata.delta_fwd_workspace(B, H, 700, dk, dv, C, 1)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    for T, seed in ((700, 6800), (130, 6801)):
        q, k, v = (dev(x, "bf16") for x in gen.gaussian_qkv(B, H, T, dk, dv, seed=seed, dtype="bf16"))
        beta = dev(_betas(B, H, T, seed + 1))
        say(f"delta workspace reuse T={T}")
        o1 = torch.empty_like(v)
        kata.delta_fwd_into(q, k, v, beta, o1, C, workspace=ws)
        o2 = kata.delta_fwd(q, k, v, beta, chunk=C)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    with pytest.raises(kata.KataError):
        kata.delta_fwd_into(q, k, v, beta, o1, C, workspace=ws[:16])
