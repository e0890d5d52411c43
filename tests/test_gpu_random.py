"""Seeded random configurations across every option of the chunked forwards (and
of the factored-feature and DeltaKATA forwards, below):
batch, heads, any length T (ragged tails, T not a multiple of 4 across heads),
d_k, d_v, chunk, dtype, feature map, prefix method, causal or not, decay gate,
initial state. Each runs through the C ABI and is compared with the float64
oracles (oracle/kata_oracle.py, oracle/first_order_oracle.py,
oracle/decay_oracle.py): outputs row-relative within 1e-4 (fp32 inputs) or
2e-2 (bf16), final states within 1e-4 where every lifted key enters the state
exactly (fp32 inputs, the fp32 path, and the gated PSD matrix-core kernels,
which take split operands) and 2e-2 elsewhere (the matrix cores round lifted
keys to bf16). Configurations are drawn only from
the supported set: the sequential prefix needs a bf16 matrix-core shape, and
the gated matrix-core shapes also T % 4 == 0 or a single head. Initial states
stand for 1-300 earlier tokens, for causal and non-causal calls alike, and
per-token decays reach down to exp(-0.5)."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, say, state_rel_err

pytestmark = pytest.mark.gpu

N_CASES = 96


def _matrix_core_shape(dtype, feature, dk, C, gated):
    if dtype != "bf16":
        return False
    if feature == "identity":
        return C in ((32, 64) if gated else (32, 64, 128))
    return (dk == 16 and C in (32, 64)) or (dk == 32 and C in (64, 128))


def _draw(i):
    r = np.random.Generator(np.random.PCG64(7000 + i))
    cfg = {
        "B": int(r.integers(1, 3)), "H": int(r.integers(1, 4)),
        "T": int(r.choice([int(r.integers(1, 9)), int(r.integers(9, 260)), int(r.integers(260, 700))])),
        "dk": int(r.choice([16, 32])), "dv": int(r.choice([16, 32, 64])),
        "C": int(r.choice([16, 32, 64, 128])), "dtype": str(r.choice(["bf16", "bf16", "f32"])),
        "feature": str(r.choice(["psd", "psd", "identity"])), "gated": bool(r.random() < 0.4),
    }
    cfg["causal"] = cfg["gated"] or bool(r.random() < 0.85)
    # an initial state standing for 1-300 earlier tokens (half of them for at
    # most 8: the few-key regime)
    cfg["S0"] = bool(r.random() < 0.5)
    cfg["T0"] = int(r.choice([int(r.integers(1, 9)), int(r.integers(1, 300))]))
    mc = _matrix_core_shape(cfg["dtype"], cfg["feature"], cfg["dk"], cfg["C"], cfg["gated"])
    if cfg["gated"] and cfg["T"] % 4 and cfg["B"] * cfg["H"] > 1:
        mc = False                              # gated matrix cores stage T-aligned rows
    cfg["mc"] = mc
    cfg["prefix"] = "sequential" if mc and r.random() < 0.4 else "scan"
    cfg["gmin"] = float(r.choice([-0.02, -0.2, -0.5]))
    return cfg


CASES = [_draw(i) for i in range(N_CASES)]


def _ids(c):
    return (f"B{c['B']}H{c['H']}T{c['T']}d{c['dk']}v{c['dv']}C{c['C']}{c['dtype']}-{c['feature']}-"
            f"{c['prefix']}{'' if c['causal'] else '-full'}{'-gated' if c['gated'] else ''}"
            f"{'-S0' if c['S0'] else ''}")


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


@pytest.mark.parametrize("c", CASES, ids=[_ids(c) for c in CASES])
def test_random_config(kata, c):
    import torch
    B, H, T, dk, dv, dtype, feature = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["dtype"], c["feature"]
    draw = gen.orthant_qkv if feature == "identity" else gen.gaussian_qkv
    T0 = c["T0"] if c["S0"] else 0
    seed = 7100 + CASES.index(c)
    q, k, v = draw(B, H, T0 + T, dk, dv, seed=seed, dtype=dtype)
    g = gen.log_decays(B, H, T0 + T, seed=seed + 1, gmin=c["gmin"]) if c["gated"] else None
    S0 = z0 = None
    if c["S0"]:
        if c["gated"]:
            _, S0, z0 = O.decay_recurrent(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], g[:, :, :T0],
                                          feature=feature)
        elif feature == "identity":
            S0, z0 = O.fo_state_from_tokens(k[:, :, :T0], v[:, :, :T0])
        else:
            S0, z0 = O.state_from_tokens(k[:, :, :T0], v[:, :, :T0])
    qs, ks, vs = q[:, :, T0:], k[:, :, T0:], v[:, :, T0:]
    say(f"random {_ids(c)}")
    init = None if S0 is None else (dev(S0.astype(np.float32)), dev(z0.astype(np.float32)))
    want_state = c["causal"]
    if c["gated"]:
        out = kata.chunked_fwd_decay(dev(qs, dtype), dev(ks, dtype), dev(vs, dtype), dev(g[:, :, T0:]),
                                     chunk=c["C"], initial_state=init, return_state=True,
                                     prefix=c["prefix"], feature=feature)
    else:
        out = kata.chunked_fwd(dev(qs, dtype), dev(ks, dtype), dev(vs, dtype), chunk=c["C"],
                               causal=c["causal"], initial_state=init, return_state=want_state,
                               feature=feature, prefix=c["prefix"])
    torch.cuda.synchronize()
    o, (S, z) = out if want_state else (out, (None, None))
    o = host(o)

    if c["gated"]:
        o_ref = O.decay_brute_force(q, k, v, g, feature=feature)[:, :, T0:]
        _, S_ref, z_ref = O.decay_recurrent(q, k, v, g, feature=feature)
    elif feature == "identity":
        o_ref = O.fo_brute_force(qs, ks, vs, causal=c["causal"], S0=S0, z0=z0)
        S_ref, z_ref = O.fo_state_from_tokens(k, v)
    else:
        o_ref = O.brute_force(qs, ks, vs, causal=c["causal"], S0=S0, z0=z0)
        S_ref, z_ref = O.state_from_tokens(k, v)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert np.all(np.isfinite(o))
    assert row_rel_err(o, o_ref) <= tol
    if want_state:
        # bf16-rounded key lifts: the matrix-core kernels without split operands
        rounded = dtype == "bf16" and c["mc"] and (feature == "identity" or not c["gated"])
        stol = 2e-2 if rounded else 1e-4
        assert state_rel_err(host(S), S_ref) <= stol and state_rel_err(host(z), z_ref) <= stol


def _draw_flash(i):
    r = np.random.Generator(np.random.PCG64(7500 + i))
    return {"B": int(r.integers(1, 3)), "H": int(r.integers(1, 4)),
            "T": int(r.choice([int(r.integers(1, 40)), int(r.integers(40, 700))])),
            "dk": int(r.choice([16, 32])), "dv": int(r.choice([16, 32, 64])),
            "causal": bool(r.random() < 0.75)}


FLASH_CASES = [_draw_flash(i) for i in range(24)]


@pytest.mark.parametrize("c", FLASH_CASES,
                         ids=[f"B{c['B']}H{c['H']}T{c['T']}d{c['dk']}v{c['dv']}{'' if c['causal'] else '-full'}"
                              for c in FLASH_CASES])
def test_random_flash(kata, c):
    """The quadratic-form forward (bf16) on random shapes against the brute force."""
    import torch
    q, k, v = gen.gaussian_qkv(c["B"], c["H"], c["T"], c["dk"], c["dv"],
                               seed=7600 + FLASH_CASES.index(c), dtype="bf16")
    say(f"random flash {c}")
    o = kata.flash_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=c["causal"])
    torch.cuda.synchronize()
    assert row_rel_err(host(o), O.brute_force(q, k, v, causal=c["causal"])) <= 2e-2


def _draw_decode(i):
    r = np.random.Generator(np.random.PCG64(7700 + i))
    return {"N": int(r.choice([1, int(r.integers(2, 64)), int(r.integers(64, 700))])),
            "dk": int(r.choice([16, 32])), "dv": int(r.choice([16, 32, 64])),
            "dtype": str(r.choice(["bf16", "f32"])), "gated": bool(r.random() < 0.5)}


DECODE_CASES = [_draw_decode(i) for i in range(24)]


@pytest.mark.parametrize("c", DECODE_CASES,
                         ids=[f"N{c['N']}d{c['dk']}v{c['dv']}{c['dtype']}{'-gated' if c['gated'] else ''}"
                              for c in DECODE_CASES])
def test_random_decode(kata, c):
    """Three decode steps from a state built from 30 earlier tokens, on random
    row counts and shapes: outputs and the updated state against the oracle's
    step (1e-5 for fp32 inputs, whose step is fp32 arithmetic; 2e-2 for bf16
    outputs, 1e-5 for the fp32 state)."""
    import torch
    N, dk, dv, dtype, steps = c["N"], c["dk"], c["dv"], c["dtype"], 3
    seed = 7800 + DECODE_CASES.index(c)
    q, k, v = gen.gaussian_qkv(1, N, steps, dk, dv, seed=seed, dtype=dtype)
    g = gen.log_decays(1, N, steps, seed=seed + 1, gmin=-0.3)
    kp, vp = gen.gaussian_qkv(1, N, 30, dk, dv, seed=seed + 2, dtype="f32")[1:]
    S_ref, z_ref = O.state_from_tokens(kp, vp)
    S_ref, z_ref = S_ref[0], z_ref[0]
    S, z = dev(S_ref), dev(z_ref)
    say(f"random decode {c}")
    for t in range(steps):
        args = (dev(q[0, :, t], dtype), dev(k[0, :, t], dtype), dev(v[0, :, t], dtype))
        if c["gated"]:
            o = kata.decode_step_decay(*args, dev(g[0, :, t]), S, z)
            o_ref, S_ref, z_ref = O.decay_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], g[0, :, t],
                                                      S_ref, z_ref)
        else:
            o = kata.decode_step(*args, S, z)
            o_ref, S_ref, z_ref = O.decode_step(q[0, :, t], k[0, :, t], v[0, :, t], S_ref, z_ref)
        torch.cuda.synchronize()
        assert row_rel_err(host(o), o_ref) <= (1e-5 if dtype == "f32" else 2e-2)
    assert state_rel_err(host(S), S_ref, lead=1) <= 1e-5
    assert state_rel_err(host(z), z_ref, lead=1) <= 1e-5


# ---- factored PSD features (KATA-Mg / KATA-Sigma-g) -------------------------------

FACTORED_SHAPES = [(16, 2, "multi"), (16, 2, "summed"), (16, 4, "multi"), (16, 4, "summed"),
                   (32, 4, "multi"), (32, 4, "summed"), (32, 2, "summed")]


def _draw_factored(i):
    r = np.random.Generator(np.random.PCG64(7900 + i))
    dk, g, kind = FACTORED_SHAPES[int(r.integers(0, len(FACTORED_SHAPES)))]
    return {"B": int(r.integers(1, 3)), "H": int(r.integers(1, 4)),
            "T": int(r.choice([int(r.integers(1, 9)), int(r.integers(9, 260)),
                               int(r.integers(260, 700)), int(r.integers(2000, 9000))])),
            "dk": dk, "g": g, "kind": kind, "dv": int(r.choice([32, 64])),
            "causal": bool(r.random() < 0.85), "S0": bool(r.random() < 0.5),
            "T0": int(r.choice([int(r.integers(1, 9)), int(r.integers(1, 300))]))}


FACTORED_CASES = [_draw_factored(i) for i in range(32)]


def _fid(c):
    return (f"B{c['B']}H{c['H']}T{c['T']}d{c['dk']}v{c['dv']}-{c['kind']}{c['g']}"
            f"{'' if c['causal'] else '-full'}{'-S0' if c['S0'] else ''}")


@pytest.mark.parametrize("c", FACTORED_CASES, ids=[_fid(c) for c in FACTORED_CASES])
def test_random_factored(kata, c):
    """kata_factored_fwd on random shapes, lengths (up to 9000 tokens: many
    segments), causality and initial states of 1-300 tokens, against the
    factored oracle: outputs within 2e-2, final states within 1e-4 (split
    operands)."""
    import torch
    B, H, T, dk, dv, g, kind = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["g"], c["kind"]
    T0 = c["T0"] if c["S0"] else 0
    seed = 8000 + FACTORED_CASES.index(c)
    q, k, v = gen.gaussian_qkv(B, H, T0 + T, dk, dv, seed=seed, dtype="bf16")
    S0 = z0 = None
    if c["S0"]:
        S0, z0 = O.factored_state_from_tokens(k[:, :, :T0], v[:, :, :T0], g, kind)
    qs, ks, vs = q[:, :, T0:], k[:, :, T0:], v[:, :, T0:]
    say(f"random factored {_fid(c)}")
    init = None if S0 is None else (dev(S0), dev(z0))
    o, (S, z) = kata.factored_fwd(dev(qs, "bf16"), dev(ks, "bf16"), dev(vs, "bf16"), g, kind,
                                  causal=c["causal"], initial_state=init, return_state=True)
    torch.cuda.synchronize()
    o = host(o)
    assert np.all(np.isfinite(o))
    if T <= 1000:
        ref = O.factored_brute_force(qs, ks, vs, g, kind, c["causal"], S0, z0)
        assert row_rel_err(o, ref) <= 2e-2
    else:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, T - 1], np.arange(0, T, 997)]))
        ref = O.factored_brute_force_rows(qs, ks, vs, rows, g, kind, c["causal"], S0, z0)
        assert row_rel_err(o[:, :, rows], ref) <= 2e-2
    S_ref, z_ref = O.factored_state_from_tokens(k, v, g, kind)
    assert state_rel_err(host(S), S_ref) <= 1e-4 and state_rel_err(host(z), z_ref) <= 1e-4


# ---- DeltaKATA ---------------------------------------------------------------------

def _draw_delta(i):
    r = np.random.Generator(np.random.PCG64(8100 + i))
    return {"B": int(r.integers(1, 3)), "H": int(r.integers(1, 3)),
            "T": int(r.choice([int(r.integers(1, 17)), int(r.integers(17, 300)), int(r.integers(300, 900))])),
            "dk": int(r.choice([16, 32])), "dv": int(r.choice([16, 32, 64])),
            "C": int(r.choice([16, 32, 64])), "dtype": str(r.choice(["bf16", "f32"])),
            "S0": bool(r.random() < 0.5), "blo": float(r.choice([0.0, 0.5, 1.0]))}


DELTA_CASES = [_draw_delta(i) for i in range(24)]


def _did(c):
    return (f"B{c['B']}H{c['H']}T{c['T']}d{c['dk']}v{c['dv']}C{c['C']}{c['dtype']}"
            f"-beta{c['blo']}{'-S0' if c['S0'] else ''}")


@pytest.mark.parametrize("c", DELTA_CASES, ids=[_did(c) for c in DELTA_CASES])
def test_random_delta(kata, c):
    """kata_delta_fwd on random shapes, lengths, chunk sizes and dtypes, write
    strengths drawn from [beta_lo, 1], with and without an initial state,
    against the delta oracle under the bars of tests/test_gpu_delta.py."""
    import torch
    from tests.test_gpu_delta import _check_rows
    B, H, T, dk, dv, C, dtype = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["C"], c["dtype"]
    seed = 8200 + DELTA_CASES.index(c)
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=seed, dtype=dtype)
    rb = np.random.Generator(np.random.PCG64(seed + 1))
    beta = rb.uniform(c["blo"], 1.0, (B, H, T)).astype(np.float32).astype(np.float64)
    S0 = z0 = None
    if c["S0"]:
        S0, z0 = O.state_from_tokens(*gen.gaussian_qkv(B, H, 5, dk, dv, seed=seed + 2, dtype="f32")[1:])
    say(f"random delta {_did(c)}")
    init = None if S0 is None else (dev(S0.astype(np.float32)), dev(z0.astype(np.float32)))
    o, (S, z) = kata.delta_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(beta), chunk=C,
                               initial_state=init, return_state=True)
    torch.cuda.synchronize()
    num, den, S_ref, z_ref = O.delta_recurrent(q, k, v, beta, S0, z0, parts=True)
    _check_rows(host(o), num, den, dtype)
    assert state_rel_err(host(S), S_ref) <= 1e-4 and state_rel_err(host(z), z_ref) <= 1e-4
