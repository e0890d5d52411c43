"""GPU parity of the quadratic (flash-style) forward, kata_flash_fwd, against the
float64 brute-force oracle: the same output the chunked form computes, reached
without chunk states, so it also cross-checks the chunked path independently.
bf16 inputs with fp32 accumulation: tolerance 2e-2 (row-normwise)."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, sample_rows, say, workload_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def run_flash(kata, q, k, v, causal=True):
    """Output buffer pre-filled with NaN: an element the kernel does not write
    cannot pass."""
    import torch
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o = torch.full_like(vd, float("nan"))
    kata.flash_fwd(qd, kd, vd, causal=causal, out=o)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("dk,dv", [(16, 64), (16, 16), (16, 32), (32, 64), (32, 32), (32, 16)])
@pytest.mark.parametrize("T", [1, 7, 64, 127, 128, 129, 1000])
def test_flash_causal(kata, dk, dv, T):
    q, k, v = gen.gaussian_qkv(2, 3, T, dk, dv, seed=700 + dk + dv + T, dtype="bf16")
    say(f"flash causal dk={dk} dv={dv} T={T}")
    o = run_flash(kata, q, k, v)
    assert row_rel_err(o, O.brute_force(q, k, v)) <= TOL
    if T == 1:   # a single token: (w v) / w rounds back to v
        assert np.array_equal(o, v.astype(np.float64))


@pytest.mark.parametrize("dk", [16, 32])
@pytest.mark.parametrize("T", [100, 333])
def test_flash_noncausal(kata, dk, T):
    q, k, v = gen.gaussian_qkv(2, 2, T, dk, 64, seed=750 + dk + T, dtype="bf16")
    say(f"flash noncausal dk={dk} T={T}")
    o = run_flash(kata, q, k, v, causal=False)
    assert row_rel_err(o, O.brute_force(q, k, v, causal=False)) <= TOL


@pytest.mark.parametrize("heads", [1, 8, 16])
def test_flash_head_mapping(kata, heads):
    """B*H a multiple of 8 takes the head-to-XCD block order, otherwise the plain
    one; every (head, query block) must be computed exactly once."""
    q, k, v = gen.gaussian_qkv(1, heads, 300, 16, 64, seed=780 + heads, dtype="bf16")
    say(f"flash heads={heads}")
    o = run_flash(kata, q, k, v)
    assert row_rel_err(o, O.brute_force(q, k, v)) <= TOL


@pytest.mark.parametrize("dk", [16, 32])
def test_flash_bitwise_causality(kata, dk):
    """Perturbing token j leaves every output before j bit-identical."""
    T = 300
    q, k, v = gen.gaussian_qkv(1, 2, T, dk, 64, seed=790 + dk, dtype="bf16")
    say(f"flash causality dk={dk}")
    base = run_flash(kata, q, k, v)
    for j in [63, 64, 127, 128, 129, 255]:
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, :, j] = gen.round_to(-q[:, :, j] + 0.25, "bf16")
        k2[:, :, j] = gen.round_to(k[:, :, j][..., ::-1] + 0.5, "bf16")
        v2[:, :, j] = gen.round_to(v[:, :, j] * 3.0 + 1.0, "bf16")
        got = run_flash(kata, q2, k2, v2)
        assert np.array_equal(got[:, :, :j], base[:, :, :j]), f"output before {j} changed"
        assert not np.array_equal(got[:, :, j], base[:, :, j])


def test_flash_zero_query_rows(kata):
    """A zero query has a zero denominator: its output row is exactly 0."""
    q, k, v = gen.gaussian_qkv(1, 1, 200, 16, 64, seed=799, dtype="bf16")
    q[:, :, 5] = 0.0
    q[:, :, 150] = 0.0
    o = run_flash(kata, q, k, v)
    assert np.all(o[:, :, 5] == 0.0) and np.all(o[:, :, 150] == 0.0)
    assert row_rel_err(o, O.brute_force(q, k, v)) <= TOL


def test_flash_deterministic(kata):
    q, k, v = gen.gaussian_qkv(2, 4, 1500, 32, 64, seed=801, dtype="bf16")
    a = run_flash(kata, q, k, v)
    b = run_flash(kata, q, k, v)
    assert np.array_equal(a, b)


def test_flash_fullsize_fwd4k(kata):
    """The 4k workload at full size: sampled rows against the oracle, and the
    chunked path's output within the same tolerance."""
    import torch
    w, q, k, v, _ = workload_inputs("fwd4k")
    say(f"flash full size fwd4k B{w.B} H{w.H} T{w.T}")
    o = run_flash(kata, q, k, v)
    assert np.all(np.isfinite(o))
    rows = sample_rows(w.T, w.chunk)
    ref = O.brute_force_rows(q, k, v, rows)
    assert row_rel_err(o[:, :, rows], ref) <= TOL
    oc = host(kata.chunked_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), chunk=w.chunk))
    torch.cuda.synchronize()
    assert row_rel_err(oc[:, :, rows], ref) <= TOL
    assert row_rel_err(o, oc) <= 2 * TOL
