"""Pins of the decay-gated float64 oracle (oracle/decay_oracle.py).

Each check takes a namespace with the decay functions and the PSD-lift oracle's
brute_force and prefix_states, so that test_decay_oracle.py can run the same
checks against copies with a planted mistake.

  no_decay          g = 0 reduces to the ungated brute force and prefix states
  golden_worked     hand-worked rationals, gamma = 1/2 (tests/golden/decay_t3.txt)
  rows_eq           the rows-only brute force = the full one on those rows
  recurrent_eq      brute force = token recurrence (with an initial state)
  chunk_invariance  chunked form with the log-depth combine scan = brute force
                    for every C; final state = the recurrence's
  combine_laws      the chunk-state operator is associative, not commutative,
                    and (1, 0, 0) is its identity
  ema_closed_form   parallel queries and keys with constant gamma: the
                    exponentially weighted mean sum gamma^(t-j) v_j / sum gamma^(t-j)
  reset             gamma = 0 at token s and no decay after it: later outputs
                    equal the ungated brute force on the suffix from s
  convexity         outputs lie in the hull of the visible values
  decode_chain      repeated decode steps = recurrence
  identity_*        the same laws with the first-order feature phi1(x) = x:
                    g = 0 gives the first-order oracle (brute force and state
                    totals), recurrence = brute force, chunk invariance, the
                    EMA closed form, the reset, the decode chain
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
    assert float(np.max(np.abs(a - b))) <= tol * scale


def _case(seed, B=2, H=2, T=17, d=3, dv=4, gmin=-1.0):
    r = _rng(seed)
    q, k, v = (r.standard_normal((B, H, T, d)), r.standard_normal((B, H, T, d)),
               r.standard_normal((B, H, T, dv)))
    g = r.uniform(gmin, 0.0, (B, H, T))
    return q, k, v, g


def _state0(O, seed, B=2, H=2, d=3, dv=4):
    r = _rng(seed)
    kp, vp = r.standard_normal((B, H, 6, d)), r.standard_normal((B, H, 6, dv))
    return O.prefix_states(kp, vp, 6)[2:]


def no_decay(O):
    q, k, v, g = _case(1)
    g[:] = 0.0
    S0, z0 = _state0(O, 2)
    _close(O.decay_brute_force(q, k, v, g), O.brute_force(q, k, v))
    _close(O.decay_brute_force(q, k, v, g, S0=S0, z0=z0), O.brute_force(q, k, v, S0=S0, z0=z0))
    P, Z, S, z = O.decay_prefix_states(k, v, g, 4)
    P2, Z2, S2, z2 = O.prefix_states(k, v, 4)
    _close(P, P2)
    _close(Z, Z2)
    _close(S, S2)


def _parse(path):
    rows = {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        rows[key] = vals
    return rows


def golden_worked(O):
    g = _parse(os.path.join(GOLDEN, "decay_t3.txt"))
    for pre, d in (("d1", 1), ("d2", 2)):
        q = np.array(g[pre + "_q"], np.float64).reshape(1, 1, 3, d)
        k = np.array(g[pre + "_k"], np.float64).reshape(1, 1, 3, d)
        v = np.array(g[pre + "_v"], np.float64).reshape(1, 1, 3, 1)
        lg = np.full((1, 1, 3), -np.log(2.0))
        want = np.array([float(Fraction(x)) for x in g[pre + "_o"]]).reshape(1, 1, 3, 1)
        _close(O.decay_brute_force(q, k, v, lg), want, 1e-14)
        _close(O.decay_recurrent(q, k, v, lg)[0], want, 1e-14)
        _close(O.decay_chunked(q, k, v, lg, 2)[0], want, 1e-14)


def rows_eq(O):
    q, k, v, g = _case(12, T=21)
    rows = [0, 3, 7, 20]
    _close(O.decay_brute_force_rows(q, k, v, g, rows), O.decay_brute_force(q, k, v, g)[:, :, rows])


def recurrent_eq(O):
    q, k, v, g = _case(3)
    S0, z0 = _state0(O, 4)
    o, S, z = O.decay_recurrent(q, k, v, g, S0=S0, z0=z0)
    _close(o, O.decay_brute_force(q, k, v, g, S0=S0, z0=z0), 1e-9)


def chunk_invariance(O):
    q, k, v, g = _case(5, T=23)
    S0, z0 = _state0(O, 6)
    ref = O.decay_brute_force(q, k, v, g, S0=S0, z0=z0)
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g, S0=S0, z0=z0)
    for C in (1, 2, 3, 5, 8, 23, 30):
        o, S, z = O.decay_chunked(q, k, v, g, C, S0=S0, z0=z0)
        _close(o, ref, 1e-9)
        _close(S, S_ref, 1e-10)
        _close(z, z_ref, 1e-10)


def combine_laws(O):
    r = _rng(7)
    mk = lambda: (r.uniform(0.1, 1.0, (2, 2)), r.standard_normal((2, 2, 3, 4)), r.standard_normal((2, 2, 3)))
    x, y, w = mk(), mk(), mk()
    lhs = O.decay_combine(O.decay_combine(x, y), w)
    rhs = O.decay_combine(x, O.decay_combine(y, w))
    for a, b in zip(lhs, rhs):
        _close(a, b)
    xy, yx = O.decay_combine(x, y), O.decay_combine(y, x)
    assert np.max(np.abs(xy[1] - yx[1])) > 1e-3          # order matters
    ident = (np.ones((2, 2)), np.zeros((2, 2, 3, 4)), np.zeros((2, 2, 3)))
    for a, b in zip(O.decay_combine(ident, x), x):
        _close(a, b)
    for a, b in zip(O.decay_combine(x, ident), x):
        _close(a, b)


def ema_closed_form(O):
    T, dv, gam = 12, 3, 0.8
    v = _rng(8).standard_normal((1, 1, T, dv))
    q = np.zeros((1, 1, T, 2))
    k = np.zeros((1, 1, T, 2))
    q[..., 0] = 1.0
    k[..., 0] = 1.0
    g = np.full((1, 1, T), np.log(gam))
    want = np.zeros((1, 1, T, dv))
    for t in range(T):
        wts = np.array([gam ** (t - j) for j in range(t + 1)])
        want[0, 0, t] = (wts[:, None] * v[0, 0, :t + 1]).sum(axis=0) / wts.sum()
    for o in (O.decay_brute_force(q, k, v, g), O.decay_recurrent(q, k, v, g)[0],
              O.decay_chunked(q, k, v, g, 5)[0]):
        _close(o, want, 1e-12)


def reset(O):
    q, k, v, g = _case(9, T=20)
    s = 11
    g[:, :, s] = -1e4                                     # gamma_s = exp(-1e4) = 0
    g[:, :, s + 1:] = 0.0                                 # no decay after the reset
    want = O.brute_force(q[:, :, s:], k[:, :, s:], v[:, :, s:])
    for o in (O.decay_brute_force(q, k, v, g), O.decay_recurrent(q, k, v, g)[0],
              O.decay_chunked(q, k, v, g, 4)[0]):
        _close(o[:, :, s:], want, 1e-10)


def convexity(O):
    q, k, v, g = _case(10, T=29)
    for o in (O.decay_brute_force(q, k, v, g), O.decay_chunked(q, k, v, g, 6)[0]):
        lo = np.minimum.accumulate(v, axis=2)
        hi = np.maximum.accumulate(v, axis=2)
        assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def decode_chain(O):
    q, k, v, g = _case(11, B=1, H=3, T=10)
    o_ref, S_ref, z_ref = O.decay_recurrent(q, k, v, g)
    D = q.shape[-1] * (q.shape[-1] + 1) // 2
    S = np.zeros((3, D, v.shape[-1]))
    z = np.zeros((3, D))
    for t in range(q.shape[2]):
        o, S, z = O.decay_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], g[0, :, t], S, z)
        _close(o, o_ref[0, :, t], 1e-10)
    _close(S, S_ref[0])
    _close(z, z_ref[0])


ID = "identity"


def _ocase(seed, **kw):
    """_case with queries and keys in the nonnegative orthant (the first-order
    feature's cone: weights q.k >= 0, denominators away from 0)."""
    q, k, v, g = _case(seed, **kw)
    return np.abs(q), np.abs(k), v, g


def _fo_state0(O, seed, B=2, H=2, d=3, dv=4):
    r = _rng(seed)
    kp, vp = np.abs(r.standard_normal((B, H, 6, d))), r.standard_normal((B, H, 6, dv))
    return O.fo_state_from_tokens(kp, vp)


def identity_no_decay(O):
    q, k, v, g = _ocase(21)
    g[:] = 0.0
    S0, z0 = _fo_state0(O, 22)
    _close(O.decay_brute_force(q, k, v, g, feature=ID), O.fo_brute_force(q, k, v))
    _close(O.decay_brute_force(q, k, v, g, S0=S0, z0=z0, feature=ID),
           O.fo_brute_force(q, k, v, S0=S0, z0=z0))
    _, _, S, z = O.decay_prefix_states(k, v, g, 4, feature=ID)
    S2, z2 = O.fo_state_from_tokens(k, v)
    _close(S, S2)
    _close(z, z2)


def identity_recurrent_eq(O):
    q, k, v, g = _ocase(23)
    S0, z0 = _fo_state0(O, 24)
    o, S, z = O.decay_recurrent(q, k, v, g, S0=S0, z0=z0, feature=ID)
    _close(o, O.decay_brute_force(q, k, v, g, S0=S0, z0=z0, feature=ID), 1e-9)
    rows = [0, 5, 16]
    _close(O.decay_brute_force_rows(q, k, v, g, rows, feature=ID),
           O.decay_brute_force(q, k, v, g, feature=ID)[:, :, rows])


def identity_chunk_invariance(O):
    q, k, v, g = _ocase(25, T=23)
    S0, z0 = _fo_state0(O, 26)
    ref = O.decay_brute_force(q, k, v, g, S0=S0, z0=z0, feature=ID)
    _, S_ref, z_ref = O.decay_recurrent(q, k, v, g, S0=S0, z0=z0, feature=ID)
    for C in (1, 3, 8, 23):
        o, S, z = O.decay_chunked(q, k, v, g, C, S0=S0, z0=z0, feature=ID)
        _close(o, ref, 1e-9)
        _close(S, S_ref, 1e-10)
        _close(z, z_ref, 1e-10)


def identity_ema(O):
    T, dv, gam = 12, 3, 0.7
    v = _rng(27).standard_normal((1, 1, T, dv))
    q = np.zeros((1, 1, T, 2))
    k = np.zeros((1, 1, T, 2))
    q[..., 1] = 1.0
    k[..., 1] = 1.0
    g = np.full((1, 1, T), np.log(gam))
    want = np.zeros((1, 1, T, dv))
    for t in range(T):
        wts = np.array([gam ** (t - j) for j in range(t + 1)])
        want[0, 0, t] = (wts[:, None] * v[0, 0, :t + 1]).sum(axis=0) / wts.sum()
    for o in (O.decay_brute_force(q, k, v, g, feature=ID), O.decay_recurrent(q, k, v, g, feature=ID)[0],
              O.decay_chunked(q, k, v, g, 5, feature=ID)[0]):
        _close(o, want, 1e-12)


def identity_reset(O):
    q, k, v, g = _ocase(28, T=20)
    s = 9
    g[:, :, s] = -1e4
    g[:, :, s + 1:] = 0.0
    want = O.fo_brute_force(q[:, :, s:], k[:, :, s:], v[:, :, s:])
    for o in (O.decay_brute_force(q, k, v, g, feature=ID), O.decay_recurrent(q, k, v, g, feature=ID)[0],
              O.decay_chunked(q, k, v, g, 4, feature=ID)[0]):
        _close(o[:, :, s:], want, 1e-10)


def identity_decode_chain(O):
    q, k, v, g = _ocase(29, B=1, H=3, T=10)
    o_ref, S_ref, z_ref = O.decay_recurrent(q, k, v, g, feature=ID)
    S = np.zeros((3, q.shape[-1], v.shape[-1]))
    z = np.zeros((3, q.shape[-1]))
    for t in range(q.shape[2]):
        o, S, z = O.decay_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], g[0, :, t], S, z, feature=ID)
        _close(o, o_ref[0, :, t], 1e-10)
    _close(S, S_ref[0])
    _close(z, z_ref[0])


ALL = [no_decay, golden_worked, rows_eq, recurrent_eq, chunk_invariance, combine_laws, ema_closed_form,
       reset, convexity, decode_chain, identity_no_decay, identity_recurrent_eq,
       identity_chunk_invariance, identity_ema, identity_reset, identity_decode_chain]


def failures(O):
    bad = []
    for chk in ALL:
        try:
            chk(O)
        except Exception:          # noqa: BLE001 - any failure counts as caught
            bad.append(chk.__name__)
    return bad
