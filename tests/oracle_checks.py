"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

Every check takes the oracle module (or a namespace with the same functions) so
that test_oracle_mutations.py can run the same checks against copies of the
oracle with a planted mistake and confirm that each mistake is caught.

What pins what (tags name the web pages on arXiv 2607.17419 and linear attention):
  phi_identity       closed form <phi(q), phi(k)> = (q.k)^2 (PSD lift, explainer 2.2)
  golden_worked      hand-worked rational outputs (tests/golden/worked_t3_d2.txt)
  golden_states      hand-worked chunk prefixes (tests/golden/worked_state_basis.txt)
  recurrent_eq       brute force = token recurrence (abstract: recurrent inference)
  chunk_invariance   brute force = chunked form for every C (abstract: "exact" form)
  convexity          outputs in the coordinatewise hull of visible values (convex gate)
  gate_identity      o_t = (1-g) r_{t-1} + g v_t (explainer 2.1: gate blends
                     previous readout with current value)
  special_cases      T=1, identical keys (prefix mean), d=1, basis keys (subset
                     means), zero query, orthogonal query, non-causal global state
  invariances        orthogonal R, per-row sign flips, scalar scaling (isometric
                     invariance, explainer 2.1)
  prefix_integer     chunk prefixes with basis keys and integer values, counted
                     independently with bincount
  decode_chain       repeated decode steps = recurrence; resume from a state
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_qkv(seed, B=2, H=2, T=19, d=3, dv=4):
    r = _rng(seed)
    return (r.standard_normal((B, H, T, d)), r.standard_normal((B, H, T, d)),
            r.standard_normal((B, H, T, dv)))


def _close(a, b, tol=1e-11):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err} > {tol * scale}"


def _parse(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        rows = [[float(Fraction(x)) for x in row.split()] for row in val.split(";")]
        out[key.strip()] = np.array(rows, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------

def phi_identity(O):
    for d in (1, 2, 3, 5, 16, 32):
        assert O.phi_dim(d) == d * (d + 1) // 2
        pairs = O.pack_pairs(d)
        assert len(pairs) == O.phi_dim(d)
        for p, (i, j) in enumerate(pairs):          # row-major upper-triangle index
            assert i <= j and p == i * d - i * (i - 1) // 2 + (j - i)
        r = _rng(d)
        x = r.standard_normal((7, d))
        y = r.standard_normal((5, d))
        fx, fy = O.phi(x), O.phi(y)
        assert fx.shape == (7, O.phi_dim(d))
        _close(fx @ fy.T, (x @ y.T) ** 2)
        # phi is the packed u u^T: its squared norm is |x|^4 and unpacking it
        # (halving off-diagonal squares) recovers the outer product entries
        _close((fx ** 2).sum(-1), (x ** 2).sum(-1) ** 2)
        M = np.zeros((7, d, d))
        for p, (i, j) in enumerate(pairs):
            s = 1.0 if i == j else 1.0 / math.sqrt(2.0)
            M[:, i, j] = M[:, j, i] = s * fx[:, p]
        _close(M, x[:, :, None] * x[:, None, :])


def golden_worked(O):
    g = _parse(os.path.join(GOLDEN, "worked_t3_d2.txt"))
    q, k, v = (g[n][None, None] for n in ("q", "k", "v"))
    _close(O.brute_force(q, k, v, causal=True)[0, 0], g["causal"], 1e-14)
    _close(O.brute_force(q, k, v, causal=False)[0, 0], g["noncausal"], 1e-14)
    for C in (1, 2, 3):
        _close(O.chunked(q, k, v, C, causal=True)[0][0, 0], g["causal"], 1e-14)
    _close(O.recurrent(q, k, v)[0][0, 0], g["causal"], 1e-14)
    _close(O.phi(g["q"][2]) @ O.phi(g["k"][1]), g["phi_k1_dot_phi_q2"][0, 0], 1e-14)


def golden_states(O):
    g = _parse(os.path.join(GOLDEN, "worked_state_basis.txt"))
    k, v = g["k"][None, None], g["v"][None, None]
    P, Z, S, z = O.prefix_states(k, v, 2)
    assert P.shape == (1, 1, 3, 3, 2) and Z.shape == (1, 1, 3, 3)
    _close(P[0, 0, 0], np.zeros((3, 2)), 0)
    _close(P[0, 0, 1], g["P1"], 0)
    _close(Z[0, 0, 1], g["Z1"][0], 0)
    _close(P[0, 0, 2], g["P2"], 0)
    _close(Z[0, 0, 2], g["Z2"][0], 0)
    _close(S[0, 0], g["final_S"], 0)
    _close(z[0, 0], g["final_z"][0], 0)


def recurrent_eq(O):
    q, k, v = _rand_qkv(11)
    ref = O.brute_force(q, k, v)
    o, S, z = O.recurrent(q, k, v)
    _close(o, ref)
    S2, z2 = O.state_from_tokens(k, v)
    _close(S, S2)
    _close(z, z2)


def chunk_invariance(O):
    q, k, v = _rand_qkv(12, T=23)
    for causal in (True, False):
        ref = O.brute_force(q, k, v, causal=causal)
        for C in range(1, q.shape[2] + 2):
            o, S, z = O.chunked(q, k, v, C, causal=causal)
            _close(o, ref)
    # with an initial state: equals brute force over the concatenated sequence
    q2, k2, v2 = _rand_qkv(13, T=9)
    S0, z0 = O.state_from_tokens(k2, v2)
    full = O.brute_force(np.concatenate([q2, q], 2), np.concatenate([k2, k], 2),
                         np.concatenate([v2, v], 2))[:, :, 9:]
    for C in (1, 4, 7, 64):
        _close(O.chunked(q, k, v, C, S0=S0, z0=z0)[0], full)
    _close(O.brute_force(q, k, v, S0=S0, z0=z0), full)
    # non-causal with an initial state: every query sees the earlier tokens and all
    # tokens of this call, i.e. non-causal attention over the concatenation
    full_nc = O.brute_force(np.concatenate([q2, q], 2), np.concatenate([k2, k], 2),
                            np.concatenate([v2, v], 2), causal=False)[:, :, 9:]
    _close(O.chunked(q, k, v, 5, causal=False, S0=S0, z0=z0)[0], full_nc)
    _close(O.brute_force(q, k, v, causal=False, S0=S0, z0=z0), full_nc)


def convexity(O):
    q, k, v = _rand_qkv(14, T=31, dv=6)
    o = O.brute_force(q, k, v)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    oc = O.chunked(q, k, v, 5)[0]
    assert np.all(oc >= lo - 1e-12) and np.all(oc <= hi + 1e-12)


def gate_identity(O):
    q, k, v = _rand_qkv(15, T=17)
    o = O.brute_force(q, k, v)
    for t in range(1, q.shape[2]):
        w = np.einsum("bhd,bhjd->bhj", q[:, :, t], k[:, :, :t + 1]) ** 2
        g = w[..., t] / w.sum(-1)
        # readout of the state before token t, with the current query
        r_prev = np.einsum("bhj,bhjn->bhn", w[..., :t], v[:, :, :t]) / w[..., :t].sum(-1)[..., None]
        _close((1 - g)[..., None] * r_prev + g[..., None] * v[:, :, t], o[:, :, t])
    # sampled rows agree with the full computation
    rows = [0, 3, 16, 7]
    _close(O.brute_force_rows(q, k, v, rows), o[:, :, rows])
    _close(O.brute_force_rows(q, k, v, rows, causal=False),
           O.brute_force(q, k, v, causal=False)[:, :, rows])


def special_cases(O):
    r = _rng(16)
    # T = 1: the output is the single value
    q, k, v = r.standard_normal((2, 3, 1, 4)), r.standard_normal((2, 3, 1, 4)), r.standard_normal((2, 3, 1, 5))
    _close(O.brute_force(q, k, v), v)
    _close(O.chunked(q, k, v, 8)[0], v)
    # identical keys: every weight equals (q.k)^2, so the output is the prefix mean
    T = 13
    q = r.standard_normal((1, 2, T, 3))
    k = np.broadcast_to(r.standard_normal((1, 2, 1, 3)), (1, 2, T, 3)).copy()
    v = r.standard_normal((1, 2, T, 4))
    mean = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    _close(O.brute_force(q, k, v), mean)
    _close(O.chunked(q, k, v, 4)[0], mean)
    # d = 1: weights q^2 k_j^2, so o_t = sum k_j^2 v_j / sum k_j^2 (q-independent)
    q = r.standard_normal((1, 1, T, 1)) + 3.0
    k = r.standard_normal((1, 1, T, 1))
    v = r.standard_normal((1, 1, T, 3))
    k2 = k[..., 0] ** 2
    ref = np.cumsum(k2[..., None] * v, axis=2) / np.cumsum(k2, axis=2)[..., None]
    _close(O.brute_force(q, k, v), ref)
    _close(O.recurrent(q, k, v)[0], ref)
    # basis keys and queries: the readout is the mean of values stored under the
    # queried key (associative-recall readout); zero where nothing matches
    d, T = 4, 20
    kid = r.integers(0, d, T)
    qid = r.integers(0, d, T)
    k = np.eye(d)[kid][None, None]
    q = np.eye(d)[qid][None, None]
    v = r.integers(-4, 5, (1, 1, T, 3)).astype(np.float64)
    ref = np.zeros((T, 3))
    for t in range(T):
        m = kid[:t + 1] == qid[t]
        if m.any():
            ref[t] = v[0, 0, :t + 1][m].mean(0)
    _close(O.brute_force(q, k, v)[0, 0], ref, 1e-15)
    _close(O.chunked(q, k, v, 3)[0][0, 0], ref, 1e-15)
    # zero query: zero denominator -> zero output
    q, k, v = _rand_qkv(17, T=6)
    q[:, :, 2] = 0.0
    o = O.brute_force(q, k, v)
    assert np.all(o[:, :, 2] == 0.0)
    assert np.all(O.chunked(q, k, v, 4)[0][:, :, 2] == 0.0)
    assert np.all(O.recurrent(q, k, v)[0][:, :, 2] == 0.0)
    # non-causal: one global state, identical rows for identical queries
    q, k, v = _rand_qkv(18, T=9)
    q[:, :, 5] = q[:, :, 1]
    o = O.brute_force(q, k, v, causal=False)
    _close(o[:, :, 5], o[:, :, 1], 1e-15)
    S, z = O.state_from_tokens(k, v)
    fq = O.phi(q)
    _close(o, np.einsum("bhtp,bhpn->bhtn", fq, S) / np.einsum("bhtp,bhp->bht", fq, z)[..., None])
    # keys orthogonal to the query contribute nothing
    q = np.zeros((1, 1, 3, 2)); q[..., 0] = 1.0
    k = np.array([[[[0.0, 1.0], [1.0, 0.0], [0.0, 2.0]]]])
    v = np.array([[[[10.0], [3.0], [7.0]]]])
    o = O.brute_force(q, k, v)[0, 0, :, 0]
    assert o[0] == 0.0 and o[1] == 3.0 and o[2] == 3.0


def invariances(O):
    q, k, v = _rand_qkv(19, T=15, d=4)
    ref = O.brute_force(q, k, v)
    Rm, _ = np.linalg.qr(_rng(20).standard_normal((4, 4)))
    _close(O.brute_force(q @ Rm.T, k @ Rm.T, v), ref, 1e-10)
    sq = np.where(_rng(21).random(q.shape[:3]) < 0.5, -1.0, 1.0)[..., None]
    sk = np.where(_rng(22).random(k.shape[:3]) < 0.5, -1.0, 1.0)[..., None]
    _close(O.brute_force(q * sq, k * sk, v), ref, 1e-12)
    _close(O.brute_force(3.7 * q, 0.2 * k, v), ref, 1e-12)
    _close(O.chunked(q @ Rm.T, 0.5 * (k @ Rm.T), v, 4)[0], ref, 1e-10)


def prefix_integer(O):
    r = _rng(23)
    B, H, T, d, dv, C = 2, 3, 29, 5, 3, 4
    kid = r.integers(0, d, (B, H, T))
    k = np.eye(d)[kid]
    v = r.integers(-9, 10, (B, H, T, dv)).astype(np.float64)
    P, Z, S, z = O.prefix_states(k, v, C)
    NC = -(-T // C)
    diag = [i * d - i * (i - 1) // 2 for i in range(d)]       # packed index of (i, i)
    for b in range(B):
        for h in range(H):
            for c in range(NC + 1):
                n = min(T, c * C)
                cnt = np.bincount(kid[b, h, :n], minlength=d).astype(np.float64)
                sums = np.zeros((d, dv))
                np.add.at(sums, kid[b, h, :n], v[b, h, :n])
                Pe = np.zeros((O.phi_dim(d), dv))
                Ze = np.zeros(O.phi_dim(d))
                Pe[diag] = sums
                Ze[diag] = cnt
                got_P = P[b, h, c] if c < NC else S[b, h]
                got_Z = Z[b, h, c] if c < NC else z[b, h]
                assert np.array_equal(got_P, Pe) and np.array_equal(got_Z, Ze)


def decode_chain(O):
    q, k, v = _rand_qkv(24, B=1, H=3, T=12)
    o_ref, S_ref, z_ref = O.recurrent(q, k, v)
    D = O.phi_dim(q.shape[-1])
    S = np.zeros((3, D, v.shape[-1]))
    z = np.zeros((3, D))
    for t in range(q.shape[2]):
        o, S, z = O.decode_step(q[0, :, t], k[0, :, t], v[0, :, t], S, z)
        _close(o, o_ref[0, :, t])
    _close(S, S_ref[0])
    _close(z, z_ref[0])
    # resume: brute force over the whole sequence = chunked prefix then decode
    o_c, S_c, z_c = O.chunked(q[:, :, :8], k[:, :, :8], v[:, :, :8], 3)
    S, z = S_c[0], z_c[0]
    for t in range(8, 12):
        o, S, z = O.decode_step(q[0, :, t], k[0, :, t], v[0, :, t], S, z)
        _close(o, o_ref[0, :, t])


ALL = [phi_identity, golden_worked, golden_states, recurrent_eq, chunk_invariance,
       convexity, gate_identity, special_cases, invariances, prefix_integer, decode_chain]


def failures(O):
    """Names of the checks that fail for oracle-like namespace O."""
    bad = []
    for chk in ALL:
        try:
            chk(O)
        except Exception:          # noqa: BLE001 - any failure counts as caught
            bad.append(chk.__name__)
    return bad
