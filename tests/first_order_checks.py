"""Pins of the first-order float64 oracle (oracle/first_order_oracle.py).

Each check takes a namespace holding the first-order functions and the PSD-lift
oracle's phi and brute_force, so that test_first_order_oracle.py can run the
same checks against copies with a planted mistake.

  feature_relation  KATA is first-order attention on the lifted vectors:
                    fo(phi(q), phi(k), v) equals the PSD-lift brute force, since
                    <phi(q), phi(k)> = (q.k)^2 (explainer 2.2); also with an
                    initial state and non-causal
  golden_worked     hand-worked rationals (tests/golden/first_order_t3_d2.txt)
  recurrent_eq      brute force = token recurrence (abstract: recurrent form)
  chunk_invariance  chunked form = brute force for every C, same final state
  prefix_mean       parallel keys and queries: o_t is the mean of v_0..v_t
  convexity         nonnegative q, k: outputs in the hull of visible values
  invariances       positive scaling of q or k and a sign flip of q cancel
  basis_states      basis keys and integer values: S, z counted with bincount
  zero_rule         zero or orthogonal queries give exactly 0
  resume            an initial state equals the tokens it stands for (causal
                    and non-causal)
"""
from __future__ import annotations

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
    assert float(np.max(np.abs(a - b))) <= tol * scale if a.size else True


def _pos_qkv(seed, B=2, H=2, T=17, d=3, dv=4):
    r = _rng(seed)
    return (np.abs(r.standard_normal((B, H, T, d))), np.abs(r.standard_normal((B, H, T, d))),
            r.standard_normal((B, H, T, dv)))


def feature_relation(O):
    r = _rng(1)
    q, k, v = (r.standard_normal((2, 2, 13, 3)), r.standard_normal((2, 2, 13, 3)),
               r.standard_normal((2, 2, 13, 2)))
    fq, fk = O.phi(q), O.phi(k)
    for causal in (True, False):
        _close(O.fo_brute_force(fq, fk, v, causal=causal), O.brute_force(q, k, v, causal=causal))
    kp, vp = r.standard_normal((2, 2, 5, 3)), r.standard_normal((2, 2, 5, 2))
    S0 = np.einsum("bhtp,bhtn->bhpn", O.phi(kp), vp)
    z0 = O.phi(kp).sum(axis=2)
    _close(O.fo_brute_force(fq, fk, v, S0=S0, z0=z0), O.brute_force(q, k, v, S0=S0, z0=z0))


def _parse(path):
    rows = {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        rows[key] = vals
    return rows


def golden_worked(O):
    g = _parse(os.path.join(GOLDEN, "first_order_t3_d2.txt"))
    q = np.array(g["q"], np.float64).reshape(1, 1, 3, 2)
    k = np.array(g["k"], np.float64).reshape(1, 1, 3, 2)
    v = np.array(g["v"], np.float64).reshape(1, 1, 3, 1)
    for mode, causal in (("causal", True), ("full", False)):
        want = np.array([float(Fraction(x)) for x in g[mode]]).reshape(1, 1, 3, 1)
        _close(O.fo_brute_force(q, k, v, causal=causal), want, 1e-15)
    o, S, z = O.fo_recurrent(q, k, v)
    _close(o, np.array([float(Fraction(x)) for x in g["causal"]]).reshape(1, 1, 3, 1), 1e-15)
    _close(S[0, 0, :, 0], np.array(g["S"], np.float64), 0)
    _close(z[0, 0], np.array(g["z"], np.float64), 0)


def recurrent_eq(O):
    for seed, signed in ((2, False), (3, True)):
        q, k, v = _pos_qkv(seed)
        if signed:
            q = q * np.where(_rng(seed + 9).random(q.shape) < 0.3, -1.0, 1.0)
        o, S, z = O.fo_recurrent(q, k, v)
        _close(o, O.fo_brute_force(q, k, v), 1e-9)
        St, zt = O.fo_state_from_tokens(k, v)
        _close(S, St)
        _close(z, zt)


def chunk_invariance(O):
    q, k, v = _pos_qkv(4, T=23)
    ref = O.fo_brute_force(q, k, v)
    St, zt = O.fo_state_from_tokens(k, v)
    for C in (1, 2, 3, 5, 8, 23, 30):
        o, S, z = O.fo_chunked(q, k, v, C)
        _close(o, ref, 1e-10)
        _close(S, St)
        _close(z, zt)
    o, S, z = O.fo_chunked(q, k, v, 4, causal=False)
    _close(o, O.fo_brute_force(q, k, v, causal=False), 1e-10)


def prefix_mean(O):
    T, dv = 9, 3
    v = _rng(5).integers(-5, 6, (1, 1, T, dv)).astype(np.float64)
    q = np.zeros((1, 1, T, 4))
    k = np.zeros((1, 1, T, 4))
    q[..., 1] = 2.5
    k[..., 1] = 0.75
    want = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    _close(O.fo_brute_force(q, k, v), want, 1e-14)
    _close(O.fo_chunked(q, k, v, 4)[0], want, 1e-14)
    _close(O.fo_brute_force(q, k, v, causal=False),
           np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), 1e-14)


def convexity(O):
    q, k, v = _pos_qkv(6, T=31)
    for o in (O.fo_brute_force(q, k, v), O.fo_recurrent(q, k, v)[0], O.fo_chunked(q, k, v, 6)[0]):
        lo = np.minimum.accumulate(v, axis=2)
        hi = np.maximum.accumulate(v, axis=2)
        assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def invariances(O):
    q, k, v = _pos_qkv(7)
    ref = O.fo_brute_force(q, k, v)
    _close(O.fo_brute_force(3.0 * q, k, v), ref, 1e-12)
    _close(O.fo_brute_force(q, 0.25 * k, v), ref, 1e-12)
    _close(O.fo_brute_force(-q, k, v), ref, 1e-12)
    # shifting v by a constant shifts every output by it (weights sum to one)
    _close(O.fo_brute_force(q, k, v + 2.0), ref + 2.0, 1e-12)


def basis_states(O):
    r = _rng(8)
    T, d, dv = 40, 5, 3
    idx = r.integers(0, d, T)
    k = np.eye(d)[idx][None, None]
    v = r.integers(-4, 5, (1, 1, T, dv)).astype(np.float64)
    S, z = O.fo_state_from_tokens(k, v)
    for a in range(d):
        for n in range(dv):
            assert S[0, 0, a, n] == np.bincount(idx, weights=v[0, 0, :, n], minlength=d)[a]
    assert np.array_equal(z[0, 0], np.bincount(idx, minlength=d).astype(np.float64))


def zero_rule(O):
    q, k, v = _pos_qkv(9, B=1, H=1, T=8, d=3)
    q[0, 0, 3] = 0.0
    k[0, 0, :, 2] = 0.0
    q[0, 0, 5] = np.array([0.0, 0.0, 1.0])      # orthogonal to every key
    for o in (O.fo_brute_force(q, k, v), O.fo_recurrent(q, k, v)[0], O.fo_chunked(q, k, v, 3)[0]):
        assert np.all(o[0, 0, 3] == 0.0) and np.all(o[0, 0, 5] == 0.0)


def resume(O):
    q, k, v = _pos_qkv(10, T=20)
    S0, z0 = O.fo_state_from_tokens(k[:, :, :7], v[:, :, :7])
    full = O.fo_brute_force(q, k, v)
    _close(O.fo_brute_force(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:], S0=S0, z0=z0), full[:, :, 7:], 1e-12)
    o, S, z = O.fo_chunked(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:], 4, S0=S0, z0=z0)
    _close(o, full[:, :, 7:], 1e-12)
    o, S2, z2 = O.fo_recurrent(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:], S0=S0, z0=z0)
    _close(o, full[:, :, 7:], 1e-10)
    St, zt = O.fo_state_from_tokens(k, v)
    _close(S, St)
    _close(S2, St)
    # non-causal: the prefix state plus every later token is every token
    full_nc = O.fo_brute_force(q, k, v, causal=False)
    for o in (O.fo_brute_force(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:], causal=False, S0=S0, z0=z0),
              O.fo_chunked(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:], 4, causal=False, S0=S0, z0=z0)[0]):
        _close(o, full_nc[:, :, 7:], 1e-12)


ALL = [feature_relation, golden_worked, recurrent_eq, chunk_invariance, prefix_mean,
       convexity, invariances, basis_states, zero_rule, resume]


def failures(O):
    bad = []
    for chk in ALL:
        try:
            chk(O)
        except Exception:          # noqa: BLE001 - any failure counts as caught
            bad.append(chk.__name__)
    return bad
