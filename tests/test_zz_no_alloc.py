"""The allocation-free forward, kata_chunked_fwd_noalloc, through the C ABI
against the workspace entry point kata_chunked_fwd on the same inputs: outputs
and final states bit-identical (the same kernels run on the same segment plan;
only where the scratch lives differs), and within the bf16 bar of the float64
oracle. Two calls in a row share the GPU's static scratch, the second on a
smaller problem; a problem larger than the scratch is refused before any
launch."""
import ctypes

import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, sample_rows, say, state_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def _call(kata, q, k, v, C, S0, z0, noalloc):
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    D = dk * (dk + 1) // 2
    nan = float("nan")
    o = torch.full_like(v, nan)
    S_out = torch.full((B, H, D, dv), nan, device="cuda")
    z_out = torch.full((B, H, D), nan, device="cuda")
    if noalloc:
        kata.chunked_fwd_noalloc_into(q, k, v, o, C, True, S0, z0, S_out, z_out)
    else:
        nbytes = kata.chunked_fwd_workspace(B, H, T, dk, dv, C, 1, True)
        assert 0 < nbytes <= kata.NOALLOC_SCRATCH_BYTES
        ws = torch.full((nbytes // 4,), nan, device="cuda")
        kata.chunked_fwd_into(q, k, v, o, C, True, ws, S0, z0, S_out, z_out)
    torch.cuda.synchronize()
    return host(o), host(S_out), host(z_out)


# first a large problem (the 131k-token shape's 39.4 MB of scratch), then
# smaller ones, so later calls meet records the earlier call left behind
CASES = [
    ("large", 1, 8, 131072, 16, 64, 64, 0),
    ("smaller", 2, 3, 1000, 32, 64, 128, 7),
    ("smallest", 1, 2, 333, 16, 32, 32, 3),
]


def test_noalloc_matches_workspace_entry_point(kata):
    for name, B, H, T, dk, dv, C, T0 in CASES:
        q, k, v = gen.gaussian_qkv(B, H, T0 + T, dk, dv, seed=9900 + T, dtype="bf16")
        S0 = z0 = None
        if T0:
            S0h, z0h = O.state_from_tokens(k[:, :, :T0], v[:, :, :T0])
            S0, z0 = dev(S0h.astype(np.float32)), dev(z0h.astype(np.float32))
        qd, kd, vd = (dev(a[:, :, T0:], "bf16") for a in (q, k, v))
        say(f"noalloc {name}: B={B} H={H} T={T} dk={dk} dv={dv} C={C} T0={T0}")
        got = _call(kata, qd, kd, vd, C, S0, z0, noalloc=True)
        ref = _call(kata, qd, kd, vd, C, S0, z0, noalloc=False)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
        o, S, z = got
        if T > 20000:                           # the oracle on sampled rows
            rows = sample_rows(T, C, n_random=8)
            o_ref = O.brute_force_rows(q[:, :2], k[:, :2], v[:, :2], rows)
            assert row_rel_err(o[:, :2, rows], o_ref) <= 2e-2
        else:
            o_ref = O.brute_force(q, k, v)[:, :, T0:]
            assert row_rel_err(o, o_ref) <= 2e-2
            S_ref, z_ref = O.state_from_tokens(k, v)
            assert state_rel_err(S, S_ref) <= 2e-2 and state_rel_err(z, z_ref) <= 2e-2


def test_noalloc_rejects_more_than_the_scratch(kata):
    """A problem whose plan needs more than the static scratch returns
    KATA_ESCRATCH before any launch (the pointers are never read)."""
    L = kata.lib()
    B, H, T = 64, 16, 131072        # 116 MB of segment records
    assert kata.chunked_fwd_workspace(B, H, T, 16, 64, 64, 1, True) > kata.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    st = L.kata_chunked_fwd_noalloc(fake, fake, fake, fake, B, H, T, 16, 64, 64, 1, 1,
                                    None, None, None, None, None)
    assert st == 5
