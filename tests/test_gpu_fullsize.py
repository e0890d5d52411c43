"""Parity at the benchmark's full sizes, in the launch configuration the
benchmark times: sampled rows against the brute-force oracle (computed one row
at a time), plus properties that hold at any size (convexity, finiteness)."""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, host, row_rel_err, sample_rows, say, state_rel_err, workload_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def _convex_ok(o, v, tol):
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    scale = np.maximum(np.abs(v).max(axis=(2, 3), keepdims=True), 1e-30)
    return np.all(o >= lo - tol * scale) and np.all(o <= hi + tol * scale)


@pytest.mark.parametrize("name", ["fwd4k", "fwd32k", "fwd131k", "recall16k"])
def test_fullsize_sampled(kata, name):
    import torch
    w, q, k, v, _ = workload_inputs(name)
    say(f"full size {name}: B{w.B} H{w.H} T{w.T} dk{w.dk} dv{w.dv} C{w.chunk}")
    o_t = kata.chunked_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), chunk=w.chunk)
    torch.cuda.synchronize()
    o = host(o_t)
    assert np.all(np.isfinite(o))
    rows = sample_rows(w.T, w.chunk)
    ref = O.brute_force_rows(q, k, v, rows)
    err = row_rel_err(o[:, :, rows], ref)
    say(f"  {name} sampled rows={rows.size} max row-rel err={err:.3e}")
    assert err <= w.tol
    assert _convex_ok(o, v.astype(np.float64), w.tol)


def test_fullsize_decode(kata):
    """Recall stream -> final states -> 1024 decode steps on 512 x 4 rows."""
    import torch
    w, q, k, v, g = workload_inputs("recall16k")
    say("decode: stream forward with state export")
    _, (S, z) = kata.chunked_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype),
                                 chunk=w.chunk, return_state=True)
    torch.cuda.synchronize()
    dq, dk, dv, src = gen.decode_continuation(g, w.H, gen.DECODE_SEQS, gen.DECODE_STEPS, seed=5000)
    N = gen.DECODE_SEQS * w.H
    S_all = S.reshape(w.B * w.H, *S.shape[2:])[torch.as_tensor(src, device="cuda")].contiguous()
    z_all = z.reshape(w.B * w.H, -1)[torch.as_tensor(src, device="cuda")].contiguous()
    S_host0 = host(S_all).astype(np.float32)
    z_host0 = host(z_all).astype(np.float32)
    dq_t, dk_t, dv_t = (dev(a.reshape(gen.DECODE_STEPS, N, -1), w.dtype) for a in (dq, dk, dv))
    outs = []
    say("decode: 1024 steps")
    for t in range(gen.DECODE_STEPS):
        outs.append(kata.decode_step(dq_t[t], dk_t[t], dv_t[t], S_all, z_all))
        if t == 0:
            torch.cuda.synchronize()
            o_ref, _, _ = O.decode_step(dq.reshape(gen.DECODE_STEPS, N, -1)[0],
                                        dk.reshape(gen.DECODE_STEPS, N, -1)[0],
                                        dv.reshape(gen.DECODE_STEPS, N, -1)[0], S_host0, z_host0)
            assert row_rel_err(host(outs[0]), o_ref) <= 2 ** -8
    torch.cuda.synchronize()
    o_all = np.stack([host(x) for x in outs])           # [steps, N, dv]
    assert np.all(np.isfinite(o_all))
    # sampled rows: brute force over the stream prefix and the decode tokens
    qf = q.reshape(w.B * w.H, w.T, -1)
    kf = k.reshape(w.B * w.H, w.T, -1)
    vf = v.reshape(w.B * w.H, w.T, -1)
    r = np.random.Generator(np.random.PCG64(1))
    for row in [0, 1, N - 1] + [int(x) for x in r.integers(0, N, 5)]:
        b = src[row]
        s, h = divmod(row, w.H)
        qq = np.concatenate([qf[b], dq[:, s, h]])[None, None]
        kk = np.concatenate([kf[b], dk[:, s, h]])[None, None]
        vv = np.concatenate([vf[b], dv[:, s, h]])[None, None]
        steps = np.arange(w.T, w.T + gen.DECODE_STEPS)
        ref = O.brute_force_rows(qq, kk, vv, steps)[0, 0]
        err = row_rel_err(o_all[:, row], ref)
        assert err <= w.tol, (row, err)


@pytest.mark.parametrize("dk,C", [(16, 64), (32, 128)])
def test_scan_states_long(kata, dk, C):
    """kata_scan_states on a 131k-token sequence (several chunks per segment,
    so the per-segment walk carries its state across chunks): sampled chunk
    prefixes, including those at segment edges, and the final state against
    the float64 sum of the tokens before them (1e-5 of the state norm)."""
    import torch
    B, H, T, dv = 1, 3, 131072 if dk == 16 else 32768, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=4400 + dk, dtype="bf16")
    say(f"scan_states long dk={dk} C={C} T={T}")
    Sp, zp, ST, zT = kata.scan_states(dev(k, "bf16"), dev(v, "bf16"), chunk=C)
    torch.cuda.synchronize()
    NC = T // C
    r = np.random.Generator(np.random.PCG64(44))
    chunks = sorted({0, 1, 2, 3, 5, 6, 7, 8, 11, 12, 13, NC // 2, NC - 2, NC - 1,
                     *(int(x) for x in r.integers(0, NC, 6))})
    for c in chunks:
        P, Z = O.state_from_tokens(k[:, :, :c * C], v[:, :, :c * C])
        assert state_rel_err(host(Sp[:, :, c]), P) <= 1e-5, c
        assert state_rel_err(host(zp[:, :, c]), Z) <= 1e-5, c
    S_ref, z_ref = O.state_from_tokens(k, v)
    assert state_rel_err(host(ST), S_ref) <= 1e-5 and state_rel_err(host(zT), z_ref) <= 1e-5
