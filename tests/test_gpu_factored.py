"""GPU parity of the factored PSD features, KATA-Mg ("multi") and KATA-Sigma-g
("summed") (kata_factored_fwd, kata_decode_step_factored), against the float64
oracle (oracle/factored_oracle.py).

Bars: outputs within 2e-2 row-relative error of the oracle (bf16 inputs with
fp32 accumulation); exported states within 1e-4 of the state norm (the lifted
keys enter the matrix cores as split bf16 operands); decode with fp32 inputs
within 1e-4; positions before a perturbed token bitwise unchanged."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, say, state_rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
STATE_TOL = 1e-4
# (d_k, g, kind) with a matrix-core kernel
SHAPES = [(16, 2, "multi"), (16, 2, "summed"), (16, 4, "multi"), (16, 4, "summed"),
          (32, 4, "multi"), (32, 4, "summed"), (32, 2, "summed")]


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def _initial(B, H, dk, dv, g, kind, n, seed):
    """A reachable initial state: the factored state of n earlier tokens."""
    _, k0, v0 = gen.gaussian_qkv(B, H, n, dk, dv, seed=seed, dtype="f32")
    return O.factored_state_from_tokens(k0, v0, g, kind)


def _run(kata, q, k, v, g, kind, causal=True, S0=None, z0=None):
    import torch
    init = None if S0 is None else (dev(S0), dev(z0))
    o, (S, z) = kata.factored_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), g, kind,
                                  chunk=64, causal=causal, initial_state=init, return_state=True)
    torch.cuda.synchronize()
    return host(o), host(S), host(z)


@pytest.mark.parametrize("dk,g,kind", SHAPES)
@pytest.mark.parametrize("dv", [32, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S0", [False, True])
def test_factored_fwd(kata, dk, g, kind, dv, causal, S0):
    """Several chunks and a ragged tail, with and without an initial state:
    every output and the exported final state."""
    B, H, T = 2, 2, 333
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=7100 + dk + 3 * g + dv, dtype="bf16")
    S0h = z0h = None
    if S0:
        S0h, z0h = _initial(B, H, dk, dv, g, kind, 9, 7101)
    say(f"factored fwd dk={dk} g={g} {kind} dv={dv} causal={causal} S0={S0}")
    o, S, z = _run(kata, q, k, v, g, kind, causal, S0h, z0h)
    ref = O.factored_brute_force(q, k, v, g, kind, causal, S0h, z0h)
    assert row_rel_err(o, ref) <= BF16_TOL
    S_ref, z_ref = O.factored_state_from_tokens(k, v, g, kind)
    if S0:
        S_ref, z_ref = S_ref + S0h, z_ref + z0h
    assert state_rel_err(S, S_ref) <= STATE_TOL and state_rel_err(z, z_ref) <= STATE_TOL


@pytest.mark.parametrize("dk,g,kind", SHAPES)
@pytest.mark.parametrize("n0", [1, 2, 3])
@pytest.mark.parametrize("T", [5, 64, 70])
def test_factored_few_key_initial_state(kata, dk, g, kind, n0, T):
    """An initial state of one to three keys: the first chunk's outputs rest on
    it alone where the chunk's own keys weigh little."""
    B, H, dv = 2, 3, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=7200 + T + n0, dtype="bf16")
    S0h, z0h = _initial(B, H, dk, dv, g, kind, n0, 7201 + n0)
    say(f"factored few-key S0 dk={dk} g={g} {kind} n0={n0} T={T}")
    for causal in (True, False):
        o, _, _ = _run(kata, q, k, v, g, kind, causal, S0h, z0h)
        assert row_rel_err(o, O.factored_brute_force(q, k, v, g, kind, causal, S0h, z0h)) <= BF16_TOL


@pytest.mark.parametrize("dk,g,kind", [(16, 2, "multi"), (16, 4, "summed"), (32, 4, "multi")])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 128, 200])
def test_factored_short_and_ragged(kata, dk, g, kind, T):
    B, H, dv = 1, 2, 32
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=7300 + T, dtype="bf16")
    say(f"factored ragged dk={dk} g={g} {kind} T={T}")
    o, S, z = _run(kata, q, k, v, g, kind)
    assert row_rel_err(o, O.factored_brute_force(q, k, v, g, kind)) <= BF16_TOL
    S_ref, z_ref = O.factored_state_from_tokens(k, v, g, kind)
    assert state_rel_err(S, S_ref) <= STATE_TOL and state_rel_err(z, z_ref) <= STATE_TOL


@pytest.mark.parametrize("dk,g,kind", [(16, 2, "multi"), (16, 2, "summed"), (32, 4, "summed")])
def test_factored_many_segments(kata, dk, g, kind):
    """Enough chunks that heads are cut into many segments of several chunks
    each (the scan over segment records), checked on sampled rows and the
    final state."""
    B, H, T, dv = 1, 2, 65536 + 37, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=7400 + dk + g, dtype="bf16")
    say(f"factored segments dk={dk} g={g} {kind} T={T}")
    o, S, z = _run(kata, q, k, v, g, kind)
    rows = np.array(sorted({0, 1, 63, 64, 65, 127, 128, 4095, 4096, 4097, 30000, T // 2,
                            T - 38, T - 37, T - 2, T - 1}))
    ref = O.factored_brute_force_rows(q, k, v, rows, g, kind)
    assert row_rel_err(o[:, :, rows], ref) <= BF16_TOL
    S_ref, z_ref = O.factored_state_from_tokens(k, v, g, kind)
    assert state_rel_err(S, S_ref) <= STATE_TOL and state_rel_err(z, z_ref) <= STATE_TOL


@pytest.mark.parametrize("dk,g,kind", [(16, 2, "multi"), (32, 4, "summed")])
def test_factored_bitwise_causality(kata, dk, g, kind):
    """A token changed at position p leaves every output before p bitwise
    unchanged (chunk-boundary and masking indices)."""
    import torch
    B, H, T, dv = 1, 2, 300, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=7500, dtype="bf16")
    base = kata.factored_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), g, kind)
    for p in (63, 64, 65, 128, 191, 299):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, p] = k[:, :, (p + 7) % T]
        v2[:, :, p] = -v[:, :, p]
        say(f"factored causality dk={dk} g={g} {kind} p={p}")
        o2 = kata.factored_fwd(dev(q, "bf16"), dev(k2, "bf16"), dev(v2, "bf16"), g, kind)
        torch.cuda.synchronize()
        assert torch.equal(base[:, :, :p], o2[:, :, :p])
        assert not torch.equal(base[:, :, p:], o2[:, :, p:])


def test_factored_g1_is_plain(kata):
    """g = 1 is the plain forward, for both kinds."""
    import torch
    B, H, T, dk, dv = 1, 2, 200, 16, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=7600, dtype="bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    say("factored g=1")
    plain = kata.chunked_fwd(qd, kd, vd)
    for kind in ("multi", "summed"):
        assert torch.equal(kata.factored_fwd(qd, kd, vd, 1, kind), plain)


def test_factored_empty_copies_initial_state(kata):
    import torch
    B, H, dk, dv, g, kind = 2, 2, 16, 64, 2, "multi"
    S0h, z0h = _initial(B, H, dk, dv, g, kind, 4, 7700)
    e = torch.empty((B, H, 0, dk), dtype=torch.bfloat16, device="cuda")
    ev = torch.empty((B, H, 0, dv), dtype=torch.bfloat16, device="cuda")
    say("factored empty")
    o, (S, z) = kata.factored_fwd(e, e, ev, g, kind, initial_state=(dev(S0h), dev(z0h)),
                                  return_state=True)
    torch.cuda.synchronize()
    assert o.shape == ev.shape
    assert np.array_equal(host(S), S0h.astype(np.float32)) and np.array_equal(host(z), z0h.astype(np.float32))


@pytest.mark.parametrize("dk,g,kind", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_factored_decode_chain(kata, dk, g, kind, dtype):
    """Decode steps from an initial state equal the recurrence."""
    import torch
    N, dv, steps = 6, 64, 5
    q, k, v = gen.gaussian_qkv(1, N, steps, dk, dv, seed=7800 + dk + g, dtype=dtype)
    S0h, z0h = _initial(1, N, dk, dv, g, kind, 3, 7801)
    o_ref, S_ref, z_ref = O.factored_recurrent(q, k, v, g, kind, S0h, z0h)
    S, z = dev(S0h[0]), dev(z0h[0])
    say(f"factored decode dk={dk} g={g} {kind} {dtype}")
    for t in range(steps):
        o = kata.decode_step_factored(dev(q[0, :, t], dtype), dev(k[0, :, t], dtype),
                                      dev(v[0, :, t], dtype), S, z, g, kind)
        torch.cuda.synchronize()
        assert row_rel_err(host(o), o_ref[0, :, t]) <= (1e-4 if dtype == "f32" else BF16_TOL)
    assert state_rel_err(host(S), S_ref[0], lead=1) <= 1e-5
    assert state_rel_err(host(z), z_ref[0], lead=1) <= 1e-5


@pytest.mark.parametrize("dk,g,kind", [(16, 2, "multi"), (16, 4, "summed")])
def test_factored_resume_then_decode(kata, dk, g, kind):
    """A prompt through the chunked forward, then decode steps from its exported
    state: the same outputs as one recurrence over prompt and new tokens."""
    import torch
    B, H, T, dv, steps = 1, 3, 200, 64, 4
    q, k, v = gen.gaussian_qkv(B, H, T + steps, dk, dv, seed=7900, dtype="bf16")
    say(f"factored resume dk={dk} g={g} {kind}")
    _, S, z = _run(kata, q[:, :, :T], k[:, :, :T], v[:, :, :T], g, kind)
    Sd, zd = dev(S[0]), dev(z[0])
    ref = O.factored_brute_force(q, k, v, g, kind)
    for t in range(T, T + steps):
        o = kata.decode_step_factored(dev(q[0, :, t], "bf16"), dev(k[0, :, t], "bf16"),
                                      dev(v[0, :, t], "bf16"), Sd, zd, g, kind)
        torch.cuda.synchronize()
        assert row_rel_err(host(o), ref[0, :, t]) <= BF16_TOL


def test_factored_fullsize_sampled(kata):
    """The fwd131k shape (B=1, H=8, T=131072, d_k=16, d_v=64, C=64) with two
    factors of width 8, both kinds, in the bench's launch configuration: sampled
    rows against the oracle one by one, and the final state."""
    from tests.gpu_util import sample_rows, workload_inputs
    w, q, k, v, _ = workload_inputs("fwd131k")
    rows = sample_rows(w.T, w.chunk, n_random=12, seed=3)
    for kind in ("multi", "summed"):
        say(f"factored fwd131k g=2 {kind}")
        o, S, z = _run(kata, q, k, v, 2, kind)
        ref = O.factored_brute_force_rows(q, k, v, rows, 2, kind)
        assert row_rel_err(o[:, :, rows], ref) <= BF16_TOL
        S_ref, z_ref = O.factored_state_from_tokens(k, v, 2, kind)
        assert state_rel_err(S, S_ref) <= STATE_TOL and state_rel_err(z, z_ref) <= STATE_TOL
