"""Pins of the DeltaKATA float64 oracle (oracle/delta_oracle.py).

Each check takes a namespace with the delta functions and the PSD-lift
oracle's brute_force, phi and state_from_tokens, so that test_delta_oracle.py
can run the same checks against copies with a planted mistake.

  golden_worked      hand-worked values (tests/golden/delta_t4_d2.txt)
  beta_zero          beta = 0 never writes: every output reads the initial
                     state (zero outputs from a zero state)
  basis_overwrite    basis-vector keys (orthonormal lifts) with beta = 1: a
                     query equal to a key returns exactly the latest value bound
                     to it - the repeated-key overwrite
  orthogonal_is_kata mutually orthogonal unit keys with beta = 1: no erase, so
                     DeltaKATA equals the plain KATA brute force
  repeated_key       one key written T times with beta = 1 and queried with
                     itself: o_t = v_t
  chunk_invariance   the chunked form equals the recurrence for every C,
                     with an initial state and random beta
  key_scale          scaling each key by a nonzero factor leaves kappa and every
                     output unchanged; scaling queries too
  rotation           rotating q and k together leaves every output unchanged
  idempotent         writing (k, v) twice with beta = 1 equals writing it once
  decode_chain       repeated decode steps equal the recurrence
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol=1e-11):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert float(np.max(np.abs(a - b))) <= tol * scale


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(seed, B=2, H=2, T=17, d=3, dv=4):
    r = _rng(seed)
    q, k, v = (r.standard_normal((B, H, T, d)), r.standard_normal((B, H, T, d)),
               r.standard_normal((B, H, T, dv)))
    beta = r.uniform(0.0, 1.0, (B, H, T))
    return q, k, v, beta


def _value(tok):
    if "sqrt2" in tok:
        num, den = tok.replace("sqrt2", "1").split("/")
        return float(eval(num)) * math.sqrt(2.0) / float(den)      # noqa: S307 - a fixture of ours
    return float(Fraction(tok))


def golden_worked(O):
    rows = {}
    for line in open(os.path.join(GOLDEN, "delta_t4_d2.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            name, *vals = line.split()
            rows[name] = np.array([_value(x) for x in vals])
    q = rows["q"].reshape(1, 1, 4, 2)
    k = rows["k"].reshape(1, 1, 4, 2)
    v = rows["v"].reshape(1, 1, 4, 1)
    b = rows["beta"].reshape(1, 1, 4)
    o, S, z = O.delta_recurrent(q, k, v, b)
    _close(o.ravel(), rows["o"], 1e-14)
    _close(S.ravel(), rows["S"], 1e-14)
    _close(z.ravel(), rows["z"], 1e-14)


def beta_zero(O):
    q, k, v, _ = _case(1)
    r = _rng(2)
    S0, z0 = O.state_from_tokens(r.standard_normal((2, 2, 5, 3)), r.standard_normal((2, 2, 5, 4)))
    o, S, z = O.delta_recurrent(q, k, v, np.zeros((2, 2, 17)), S0, z0)
    fq = O.phi(q)
    want = (fq @ S0) / (fq @ z0[..., None])
    _close(o, want)
    _close(S, S0, 0.0)
    _close(z, z0, 0.0)
    o0, _, _ = O.delta_recurrent(q, k, v, np.zeros((2, 2, 17)))
    assert np.all(o0 == 0.0)


def basis_overwrite(O):
    r = _rng(3)
    d, T, dv = 4, 40, 3
    ids = r.integers(0, d, T)
    k = np.eye(d)[ids][None, None]
    v = r.standard_normal((1, 1, T, dv))
    qi = ids.copy()
    for t in range(T):                      # query a key written at or before t
        qi[t] = ids[r.integers(0, t + 1)]
    q = np.eye(d)[qi][None, None]
    o, _, _ = O.delta_recurrent(q, k, v, np.ones((1, 1, T)))
    for t in range(T):
        last = max(j for j in range(t + 1) if ids[j] == qi[t])
        _close(o[0, 0, t], v[0, 0, last], 1e-14)


def orthogonal_is_kata(O):
    r = _rng(4)
    d, T = 6, 6
    Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
    k = Qm[None, None]                      # rows: orthonormal keys
    q = r.standard_normal((1, 1, T, d))
    v = r.standard_normal((1, 1, T, 2))
    o, S, z = O.delta_recurrent(q, k, v, np.ones((1, 1, T)))
    _close(o, O.brute_force(q, k, v))
    S_ref, z_ref = O.state_from_tokens(k, v)
    _close(S, S_ref)
    _close(z, z_ref)


def repeated_key(O):
    r = _rng(5)
    T = 12
    k = np.repeat(_unit(r.standard_normal((1, 1, 1, 3))), T, axis=2) * 1.7
    v = r.standard_normal((1, 1, T, 2))
    o, _, _ = O.delta_recurrent(k, k, v, np.ones((1, 1, T)))
    _close(o, v)


def chunk_invariance(O):
    q, k, v, b = _case(6)
    r = _rng(7)
    S0, z0 = O.state_from_tokens(r.standard_normal((2, 2, 5, 3)), r.standard_normal((2, 2, 5, 4)))
    o, S, z = O.delta_recurrent(q, k, v, b, S0, z0)
    for C in range(1, 19):
        oc, Sc, zc = O.delta_chunked(q, k, v, b, C, S0, z0)
        _close(oc, o, 1e-9)
        _close(Sc, S, 1e-10)
        _close(zc, z, 1e-10)


def key_scale(O):
    q, k, v, b = _case(8)
    o, _, _ = O.delta_recurrent(q, k, v, b)
    s = _rng(9).uniform(0.3, 3.0, k.shape[:-1] + (1,)) * np.sign(_rng(10).standard_normal(k.shape[:-1] + (1,)))
    o2, _, _ = O.delta_recurrent(q * 2.5, k * s, v, b)
    _close(o2, o, 1e-9)


def rotation(O):
    q, k, v, b = _case(11)
    R, _ = np.linalg.qr(_rng(12).standard_normal((3, 3)))
    o, _, _ = O.delta_recurrent(q, k, v, b)
    o2, _, _ = O.delta_recurrent(q @ R.T, k @ R.T, v, b)
    _close(o2, o, 1e-9)


def idempotent(O):
    r = _rng(13)
    k = r.standard_normal((1, 1, 1, 3))
    v = r.standard_normal((1, 1, 1, 2))
    q = r.standard_normal((1, 1, 1, 3))
    _, S1, z1 = O.delta_recurrent(q, k, v, np.ones((1, 1, 1)))
    _, S2, z2 = O.delta_recurrent(np.repeat(q, 2, 2), np.repeat(k, 2, 2), np.repeat(v, 2, 2),
                                  np.ones((1, 1, 2)))
    _close(S2, S1)
    _close(z2, z1)


def decode_chain(O):
    q, k, v, b = _case(14, B=1, H=3, T=6)
    o, S, z = O.delta_recurrent(q, k, v, b)
    Sd = np.zeros_like(S[0])
    zd = np.zeros_like(z[0])
    for t in range(6):
        od, Sd, zd = O.delta_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], b[0, :, t], Sd, zd)
        _close(od, o[0, :, t])
    _close(Sd, S[0])
    _close(zd, z[0])


ALL = [golden_worked, beta_zero, basis_overwrite, orthogonal_is_kata, repeated_key,
       chunk_invariance, key_scale, rotation, idempotent, decode_chain]


def failures(O):
    bad = []
    for chk in ALL:
        try:
            chk(O)
        except Exception:          # noqa: BLE001 - any failure counts as caught
            bad.append(chk.__name__)
    return bad
