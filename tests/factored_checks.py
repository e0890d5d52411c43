"""Pins of the factored-PSD oracle (oracle/factored_oracle.py): KATA-Mg
("multi") and KATA-Sigma-g ("summed").

Each check takes a namespace with the factored functions and the plain-lift
oracle's phi, brute_force and state_from_tokens (pinned on their own), so that
test_factored_oracle.py can run the same checks against copies with a planted
mistake.

  golden_worked      hand-worked values (tests/golden/factored_t3_d4.txt)
  one_factor_is_kata g = 1: both variants are the plain lift, feature and output
  feature_matrix     each packed feature unpacks to diag(x_a x_a^T) (multi) or
                     sum_a x_a x_a^T (summed), built with np.outer
  weights_are_products  phi(q).phi(k) equals the weights from the factors' dot
                     products (two independent computations)
  multi_state_blocks the multi state is the plain states of the factors, side
                     by side; the summed state is their sum
  multi_one_factor   keys living in one factor: multi is the plain KATA of that
                     factor
  summed_equal_factors  queries (u, u, ..) and keys (w, w, ..): summed is the
                     plain KATA of (u, w)
  factor_permutation summed is unchanged when each key's factors are permuted;
                     multi only when queries and keys are permuted together
  recurrent_is_brute the recurrence equals the definition, with an initial state
  chunk_invariance   the chunked form equals the definition for every C, causal
                     and not, with an initial state
  convexity          every output lies within the range of the visible values
  decode_chain       repeated decode steps equal the recurrence
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
KINDS = ("multi", "summed")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol=1e-11):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert float(np.max(np.abs(a - b))) <= tol * scale


def _value(tok):
    if "sqrt2" in tok:
        num, den = tok.replace("sqrt2", "1").split("/")
        return float(eval(num)) * math.sqrt(2.0) / float(den)      # noqa: S307 - a fixture of ours
    return float(Fraction(tok))


def _case(seed, B=2, H=2, T=13, d=8, dv=3):
    r = _rng(seed)
    return (r.standard_normal((B, H, T, d)), r.standard_normal((B, H, T, d)),
            r.standard_normal((B, H, T, dv)))


def golden_worked(O):
    rows = {}
    for line in open(os.path.join(GOLDEN, "factored_t3_d4.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            name, *vals = line.split()
            rows[name] = np.array([_value(x) for x in vals])
    q = rows["q"].reshape(1, 1, 3, 4)
    k = rows["k"].reshape(1, 1, 3, 4)
    v = rows["v"].reshape(1, 1, 3, 1)
    for kind in KINDS:
        _close(O.factored_brute_force(q, k, v, 2, kind).ravel(), rows[f"{kind}_o"], 1e-14)
        o, S, z = O.factored_recurrent(q, k, v, 2, kind)
        _close(o.ravel(), rows[f"{kind}_o"], 1e-14)
        _close(S.ravel(), rows[f"{kind}_S"], 1e-14)
        _close(z.ravel(), rows[f"{kind}_z"], 1e-14)
    _close(O.brute_force(q, k, v)[0, 0, 2, 0], rows["plain_o2"][0], 1e-14)


def one_factor_is_kata(O):
    q, k, v = _case(1, d=5)
    for kind in KINDS:
        assert O.factored_dim(5, 1, kind) == 15
        _close(O.factored_phi(q, 1, kind), O.phi(q), 0.0)
        _close(O.factored_brute_force(q, k, v, 1, kind), O.brute_force(q, k, v), 1e-12)


def _unpack(f, p):
    """Packed lift (row-major upper triangle, sqrt2 off the diagonal) -> p x p."""
    m = np.zeros((p, p))
    idx = 0
    for i in range(p):
        for j in range(i, p):
            val = f[idx] if i == j else f[idx] / math.sqrt(2.0)
            m[i, j] = m[j, i] = val
            idx += 1
    return m


def feature_matrix(O):
    r = _rng(2)
    for d, g in ((8, 2), (8, 4), (6, 3), (4, 4)):
        p = d // g
        P = p * (p + 1) // 2
        x = r.standard_normal(d)
        fm = O.factored_phi(x, g, "multi")
        assert fm.shape == (g * P,) and O.factored_dim(d, g, "multi") == g * P
        for a in range(g):
            xa = x[a * p:(a + 1) * p]
            _close(_unpack(fm[a * P:(a + 1) * P], p), np.outer(xa, xa), 1e-14)
        fs = O.factored_phi(x, g, "summed")
        assert fs.shape == (P,) and O.factored_dim(d, g, "summed") == P
        want = sum(np.outer(x[a * p:(a + 1) * p], x[a * p:(a + 1) * p]) for a in range(g))
        _close(_unpack(fs, p), want, 1e-14)


def weights_are_products(O):
    q, k, _ = _case(3, T=9, d=12)
    for g in (1, 2, 3, 4, 6):
        for kind in KINDS:
            fq = O.factored_phi(q, g, kind)
            fk = O.factored_phi(k, g, kind)
            w = O.factored_weights(q, k, g, kind)
            _close(np.einsum("bhtp,bhjp->bhtj", fq, fk), w, 1e-12)
            assert np.all(w >= 0.0)


def multi_state_blocks(O):
    _, k, v = _case(4, d=8)
    g, p = 4, 2
    Sm, zm = O.factored_state_from_tokens(k, v, g, "multi")
    Ss, zs = O.factored_state_from_tokens(k, v, g, "summed")
    parts = [O.state_from_tokens(k[..., a * p:(a + 1) * p], v) for a in range(g)]
    _close(Sm, np.concatenate([s for s, _ in parts], axis=2), 1e-12)
    _close(zm, np.concatenate([z for _, z in parts], axis=2), 1e-12)
    _close(Ss, sum(s for s, _ in parts), 1e-12)
    _close(zs, sum(z for _, z in parts), 1e-12)


def multi_one_factor(O):
    q, k, v = _case(5, d=8)
    g, p, a = 2, 4, 1
    k1 = np.zeros_like(k)
    k1[..., a * p:(a + 1) * p] = k[..., a * p:(a + 1) * p]
    want = O.brute_force(q[..., a * p:(a + 1) * p], k[..., a * p:(a + 1) * p], v)
    _close(O.factored_brute_force(q, k1, v, g, "multi"), want, 1e-12)


def summed_equal_factors(O):
    r = _rng(6)
    u = r.standard_normal((2, 2, 11, 3))
    w = r.standard_normal((2, 2, 11, 3))
    v = r.standard_normal((2, 2, 11, 4))
    for g in (2, 3):
        got = O.factored_brute_force(np.concatenate([u] * g, -1), np.concatenate([w] * g, -1), v,
                                     g, "summed")
        _close(got, O.brute_force(u, w, v), 1e-12)


def factor_permutation(O):
    r = _rng(7)
    q, k, v = _case(8, d=9)
    g, p = 3, 3
    kp = k.reshape(k.shape[:-1] + (g, p)).copy()
    for idx in np.ndindex(*kp.shape[:-2]):
        kp[idx] = kp[idx][r.permutation(g)]
    kp = kp.reshape(k.shape)
    base_s = O.factored_brute_force(q, k, v, g, "summed")
    _close(O.factored_brute_force(q, kp, v, g, "summed"), base_s, 1e-12)
    base_m = O.factored_brute_force(q, k, v, g, "multi")
    assert float(np.max(np.abs(O.factored_brute_force(q, kp, v, g, "multi") - base_m))) > 1e-3
    perm = r.permutation(g)
    joint = lambda x: x.reshape(x.shape[:-1] + (g, p))[..., perm, :].reshape(x.shape)   # noqa: E731
    _close(O.factored_brute_force(joint(q), joint(k), v, g, "multi"), base_m, 1e-12)


def _initial(O, seed, B, H, d, dv, g, kind, n=5):
    """A reachable initial state: the state of n earlier random tokens."""
    r = _rng(seed)
    return O.factored_state_from_tokens(r.standard_normal((B, H, n, d)),
                                        r.standard_normal((B, H, n, dv)), g, kind)


def recurrent_is_brute(O):
    q, k, v = _case(9, d=8)
    for g in (2, 4):
        for kind in KINDS:
            S0, z0 = _initial(O, 10, 2, 2, 8, 3, g, kind)
            o, S, z = O.factored_recurrent(q, k, v, g, kind, S0, z0)
            _close(o, O.factored_brute_force(q, k, v, g, kind, True, S0, z0), 1e-11)
            St, zt = O.factored_state_from_tokens(k, v, g, kind)
            _close(S, St + S0, 1e-11)
            _close(z, zt + z0, 1e-11)


def chunk_invariance(O):
    q, k, v = _case(11, T=10, d=8)
    for g in (2, 4):
        for kind in KINDS:
            S0, z0 = _initial(O, 12, 2, 2, 8, 3, g, kind)
            for causal in (True, False):
                want = O.factored_brute_force(q, k, v, g, kind, causal, S0, z0)
                for C in range(1, 12):
                    o, S, z = O.factored_chunked(q, k, v, C, g, kind, causal, S0, z0)
                    _close(o, want, 1e-11)
                    St, zt = O.factored_state_from_tokens(k, v, g, kind)
                    _close(S, St + S0, 1e-11)
                    _close(z, zt + z0, 1e-11)


def convexity(O):
    q, k, v = _case(13, T=40, d=8, dv=2)
    for g in (2, 4):
        for kind in KINDS:
            o = O.factored_brute_force(q, k, v, g, kind)
            lo = np.minimum.accumulate(v, axis=2)
            hi = np.maximum.accumulate(v, axis=2)
            assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def decode_chain(O):
    q, k, v = _case(14, B=1, H=3, T=7, d=8)
    for g in (2, 4):
        for kind in KINDS:
            S0, z0 = _initial(O, 15, 1, 3, 8, 3, g, kind)
            o_ref, S_ref, z_ref = O.factored_recurrent(q, k, v, g, kind, S0, z0)
            S, z = S0[0], z0[0]
            for t in range(7):
                o, S, z = O.factored_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], S, z, g, kind)
                _close(o, o_ref[0, :, t], 1e-11)
            _close(S, S_ref[0], 1e-11)
            _close(z, z_ref[0], 1e-11)


ALL = [golden_worked, one_factor_is_kata, feature_matrix, weights_are_products,
       multi_state_blocks, multi_one_factor, summed_equal_factors, factor_permutation,
       recurrent_is_brute, chunk_invariance, convexity, decode_chain]


def failures(O):
    """Names of the checks that fail for the namespace O."""
    out = []
    for check in ALL:
        try:
            check(O)
        except Exception:                                          # noqa: BLE001 - any failure counts
            out.append(check.__name__)
    return out
