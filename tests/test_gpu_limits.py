"""Parity at the largest shapes the boundary accepts along the axes that set
launch grids: B*H = 65535 heads (the largest second grid dimension; every
chunked kernel runs one grid row per head) for the matrix-core forward with
state export, the decay-gated forward, the fp32 forward and the quadratic
form. Ragged last chunks throughout. Sampled heads (first, last and random)
are checked against the float64 oracle; every output is checked for
finiteness."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, say, state_rel_err

pytestmark = pytest.mark.gpu

MAX_HEADS = 65535


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def _heads(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.integers(0, n, 8)]))


def test_max_heads_chunked_with_export(kata):
    import torch
    T, dk, dv, C = 96, 16, 16, 64
    q, k, v = gen.gaussian_qkv(1, MAX_HEADS, T, dk, dv, seed=1600, dtype="bf16")
    say(f"max heads chunked: H={MAX_HEADS} T={T}")
    o, (S, z) = kata.chunked_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), chunk=C,
                                 return_state=True)
    torch.cuda.synchronize()
    o, S, z = host(o), host(S), host(z)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)) and np.all(np.isfinite(z))
    hs = _heads(MAX_HEADS, 1601)
    assert row_rel_err(o[:, hs], O.brute_force(q[:, hs], k[:, hs], v[:, hs])) <= 2e-2
    S_ref, z_ref = O.state_from_tokens(k[:, hs], v[:, hs])
    assert state_rel_err(S[:, hs], S_ref) <= 2e-2 and state_rel_err(z[:, hs], z_ref) <= 2e-2


def test_max_heads_decay(kata):
    import torch
    T, dk, dv, C = 96, 16, 16, 32
    q, k, v = gen.gaussian_qkv(1, MAX_HEADS, T, dk, dv, seed=1610, dtype="bf16")
    g = gen.log_decays(1, MAX_HEADS, T, seed=1611, gmin=-0.2)
    say(f"max heads decay: H={MAX_HEADS} T={T}")
    o = host(kata.chunked_fwd_decay(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"),
                                    dev(g), chunk=C))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(o))
    hs = _heads(MAX_HEADS, 1612)
    assert row_rel_err(o[:, hs], O.decay_brute_force(q[:, hs], k[:, hs], v[:, hs], g[:, hs])) <= 2e-2


def test_max_heads_fp32_valu(kata):
    import torch
    T, dk, dv, C = 40, 16, 16, 16
    q, k, v = gen.gaussian_qkv(1, MAX_HEADS, T, dk, dv, seed=1620, dtype="f32")
    say(f"max heads fp32: H={MAX_HEADS} T={T}")
    o = host(kata.chunked_fwd(dev(q, "f32"), dev(k, "f32"), dev(v, "f32"), chunk=C))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(o))
    hs = _heads(MAX_HEADS, 1621)
    assert row_rel_err(o[:, hs], O.brute_force(q[:, hs], k[:, hs], v[:, hs])) <= 1e-4


def test_max_heads_flash(kata):
    import torch
    T, dk, dv = 70, 16, 16
    q, k, v = gen.gaussian_qkv(1, MAX_HEADS, T, dk, dv, seed=1630, dtype="bf16")
    say(f"max heads flash: H={MAX_HEADS} T={T}")
    o = host(kata.flash_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(o))
    hs = _heads(MAX_HEADS, 1631)
    assert row_rel_err(o[:, hs], O.brute_force(q[:, hs], k[:, hs], v[:, hs])) <= 2e-2
