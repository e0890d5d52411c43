"""The log-depth prefix (KATA_PREFIX_TREE): a Kogge-Stone scan within tiles of
128 segment (or chunk) states and reduce-then-scan across tiles. Parity with
the float64 oracles for one, two and three levels of tiles, with and without
the decay gate, on the matrix-core and fp32 paths; and the same outputs as the
blocked scan up to fp32 summation order."""
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


@pytest.mark.parametrize("dk,C,G,T", [(16, 64, 1, 300 * 64 + 17), (16, 32, 2, 130 * 64),
                                      (32, 128, 1, 140 * 128 - 5), (32, 64, 0, 3000),
                                      (16, 64, 0, 1000)])
@pytest.mark.parametrize("S0", [False, True])
def test_tree_forward(kata, dk, C, G, T, S0):
    """Segment counts below and above one tile of 128 (G = 1 gives a segment
    per chunk), an initial state, the exported final state."""
    import torch
    B, H, dv = 1, 2, 64
    T0 = 40 if S0 else 0
    q, k, v = gen.gaussian_qkv(B, H, T0 + T, dk, dv, seed=8100 + dk + C + G, dtype="bf16")
    init = None
    if S0:
        S0h, z0h = O.state_from_tokens(k[:, :, :T0], v[:, :, :T0])
        init = (dev(S0h.astype(np.float32)), dev(z0h.astype(np.float32)))
    say(f"tree forward dk={dk} C={C} G={G} T={T} S0={S0}")
    o, (S, z) = kata.chunked_fwd(dev(q[:, :, T0:], "bf16"), dev(k[:, :, T0:], "bf16"),
                                 dev(v[:, :, T0:], "bf16"), chunk=C, prefix="tree",
                                 segment_chunks=G, initial_state=init, return_state=True)
    torch.cuda.synchronize()
    rows = sample_rows(T, C, n_random=40)
    ref = O.brute_force_rows(q, k, v, rows + T0)
    assert row_rel_err(host(o)[:, :, rows], ref) <= 2e-2
    S_ref, z_ref = O.state_from_tokens(k, v)
    assert state_rel_err(host(S), S_ref) <= 2e-2 and state_rel_err(host(z), z_ref) <= 2e-2
    o2 = kata.chunked_fwd(dev(q[:, :, T0:], "bf16"), dev(k[:, :, T0:], "bf16"),
                          dev(v[:, :, T0:], "bf16"), chunk=C, prefix="scan",
                          segment_chunks=G, initial_state=init)
    torch.cuda.synchronize()
    assert row_rel_err(host(o), host(o2)) <= 2 ** -7


def test_tree_three_levels(kata):
    """16,400 segments (one chunk each): tiles of tiles of tiles."""
    import torch
    B, H, T, dk, dv, C = 1, 1, 16400 * 32, 16, 16, 32
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=8200, dtype="bf16")
    # one chunk per segment, then 16,400 -> 129 -> 2 tiles: 7 + 7 + 1 Kogge-Stone
    # levels, the init combine and one apply per level of tiles
    assert kata.prefix_depth(B, H, T, dk, dv, C, prefix="tree", segment_chunks=1) == 1 + 7 + 7 + 1 + 1 + 1 + 1
    say("tree three levels")
    o, (S, z) = kata.chunked_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), chunk=C,
                                 prefix="tree", segment_chunks=1, return_state=True)
    torch.cuda.synchronize()
    rows = sample_rows(T, 128 * C, n_random=30)
    assert row_rel_err(host(o)[:, :, rows], O.brute_force_rows(q, k, v, rows)) <= 2e-2
    S_ref, z_ref = O.state_from_tokens(k, v)
    assert state_rel_err(host(S), S_ref) <= 2e-2 and state_rel_err(host(z), z_ref) <= 2e-2


@pytest.mark.parametrize("dk,C", [(16, 64), (32, 64)])
@pytest.mark.parametrize("gmin", [-0.05, -0.5])
def test_tree_gated(kata, dk, C, gmin):
    """The tree under the decay operator (A1, S1) o (A2, S2) = (A1 A2, A2 S1 + S2):
    130 segments of one chunk (two tile levels), segment decays scanned beside
    the states, each record's tile-local decay applied to its tile's offset, an
    initial state decaying with the sequence."""
    import torch
    B, H, T, dv = 1, 1, 130 * C, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=8300 + dk, dtype="bf16")
    g = gen.log_decays(B, H, T, seed=8301, gmin=gmin)
    S0h, z0h = O.state_from_tokens(*gen.gaussian_qkv(B, H, 20, dk, dv, seed=8302, dtype="f32")[1:])
    say(f"tree gated dk={dk} C={C} gmin={gmin}")
    o, (S, z) = kata.chunked_fwd_decay(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g),
                                       chunk=C, prefix="tree", segment_chunks=1,
                                       initial_state=(dev(S0h.astype(np.float32)),
                                                      dev(z0h.astype(np.float32))),
                                       return_state=True)
    torch.cuda.synchronize()
    ref = O.decay_brute_force(q, k, v, g, S0=S0h, z0=z0h)
    assert row_rel_err(host(o), ref) <= 2e-2
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g, S0=S0h, z0=z0h)
    assert state_rel_err(host(S), S_ref) <= 1e-4 and state_rel_err(host(z), z_ref) <= 1e-4


@pytest.mark.parametrize("feature", ["psd", "identity"])
@pytest.mark.parametrize("causal", [True, False])
def test_tree_fp32_path(kata, feature, causal):
    """fp32 inputs: the tree over one state per chunk (300 chunks: two tile
    levels), fp32 arithmetic throughout."""
    import torch
    B, H, T, dk, dv, C = 1, 2, 300 * 16 + 5, 16, 16, 16
    draw = gen.orthant_qkv if feature == "identity" else gen.gaussian_qkv
    q, k, v = draw(B, H, T, dk, dv, seed=8400, dtype="f32")
    say(f"tree fp32 {feature} causal={causal}")
    out = kata.chunked_fwd(dev(q), dev(k), dev(v), chunk=C, causal=causal, prefix="tree",
                           feature=feature, return_state=causal)
    torch.cuda.synchronize()
    o, (S, z) = out if causal else (out, (None, None))
    if feature == "psd":
        ref = O.brute_force(q, k, v, causal=causal)
        S_ref, z_ref = O.state_from_tokens(k, v)
    else:
        ref = O.fo_brute_force(q, k, v, causal=causal)
        S_ref, z_ref = O.fo_state_from_tokens(k, v)
    assert row_rel_err(host(o), ref) <= 1e-4
    if causal:
        assert state_rel_err(host(S), S_ref) <= 1e-4 and state_rel_err(host(z), z_ref) <= 1e-4


def test_tree_noncausal(kata):
    """Non-causal on the matrix cores: the tree's inclusive total is the state
    every query reads."""
    import torch
    q, k, v = gen.gaussian_qkv(2, 2, 150 * 64, 16, 64, seed=8500, dtype="bf16")
    say("tree noncausal")
    o = kata.chunked_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), chunk=64, causal=False,
                         prefix="tree", segment_chunks=1)
    torch.cuda.synchronize()
    rows = sample_rows(150 * 64, 64, n_random=30)
    assert row_rel_err(host(o)[:, :, rows], O.brute_force_rows(q, k, v, rows, causal=False)) <= 2e-2
