"""Plain float64 CPU oracle for the factored PSD variants KATA-Mg and KATA-Sigma-g.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or call this module. The library (the HIP path behind
the C ABI) never does, and this module imports nothing from the library.

Sources (web pages describing arXiv 2607.17419, "Kernelized Linear Attention:
Breaking the Capacity Wall with Symmetric Cones"):

  [JA]   gist.science Japanese explainer, technical summary: 2.2 (the rank-one
         PSD lift psi(u) = u u^T squares the inner product), 2.3 "Variants"
         (KATA-Mg with multiple PSD factors and KATA-Sigma-g with summed PSD
         factors, which trade state size against packing efficiency), 4 (the
         KATA-M1 and KATA-M2 instances; M1 has the larger capacity)
  [IT]   gist.science Italian explainer, the same sections
  [LA]   notes.yuuk.io wiki page on linear attention, "Definition" (the
         normalised kernelised form)

The pages name the two variants and what they are for, and print no
construction. Reading taken (listed in the design notes): a query or key x of
width d is cut into g contiguous factors x_a = x[a p : (a + 1) p] of width
p = d / g, and each factor gives the rank-one PSD matrix x_a x_a^T of [JA 2.2].

* KATA-Mg keeps the g factors apart: the feature is the block-diagonal PSD
  matrix diag(x_1 x_1^T, ..., x_g x_g^T), packed as the g packed lifts of the
  factors one after the other (g p (p + 1) / 2 entries). Two such features
  have the Frobenius product sum_a (q_a . k_a)^2.
* KATA-Sigma-g sums the g factors into one p x p PSD matrix
  X X^T = sum_a x_a x_a^T (X = [x_1 ... x_g]), packed like a single lift
  (p (p + 1) / 2 entries). Two such features have the Frobenius product
  sum_{a,b} (q_a . k_b)^2 = |Q^T K|_F^2.

Both weights are sums of squares, so nonnegative, and with g = 1 both are the
plain KATA weight (q . k)^2; the state shrinks as g grows (about d^2 / (2 g)
features for Mg, d^2 / (2 g^2) for Sigma-g), which is the state-size /
packing trade of [JA 2.3]. The attention itself is unchanged [LA; JA 2.1]:
o_t = sum_j w_tj v_j / sum_j w_tj over j <= t (causal) or every j, zero where
the denominator is zero; the recurrent, chunked-state and decode forms are
those of the plain feature with phi replaced by the factored feature.

Parity pins: tests/factored_checks.py (run by tests/test_factored_oracle.py with
a planted-mistake suite). None of these functions is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .kata_oracle import _safe_ratio, phi, phi_dim

__all__ = [
    "FACTOR_KINDS", "factored_dim", "factored_phi", "factored_weights",
    "factored_brute_force", "factored_brute_force_rows", "factored_recurrent",
    "factored_state_from_tokens", "factored_chunked", "factored_decode_step",
]

# "multi": KATA-Mg (factors kept apart); "summed": KATA-Sigma-g (factors summed)
FACTOR_KINDS = ("multi", "summed")


def _check(d: int, g: int, kind: str) -> int:
    if kind not in FACTOR_KINDS:
        raise ValueError(f"kind must be one of {FACTOR_KINDS}, got {kind!r}")
    if g < 1 or d % g:
        raise ValueError(f"g = {g} must divide d = {d}")
    return d // g


def factored_dim(d: int, g: int, kind: str) -> int:
    """Packed feature width: g p(p+1)/2 (multi) or p(p+1)/2 (summed), p = d/g."""
    p = _check(d, g, kind)
    return g * phi_dim(p) if kind == "multi" else phi_dim(p)


def _factors(x, g: int):
    """x [..., d] -> [..., g, p]: the g contiguous factors of the last axis."""
    x = np.asarray(x, np.float64)
    return x.reshape(x.shape[:-1] + (g, x.shape[-1] // g))


def factored_phi(x, g: int, kind: str) -> np.ndarray:
    """Packed factored feature of the last axis, x [..., d] -> [..., D].

    multi: the packed lifts of the factors concatenated (factor a at entries
    [a P, (a + 1) P), P = p(p+1)/2); summed: the sum of the packed lifts of the
    factors, i.e. the packing of sum_a x_a x_a^T. Packing of one lift as for
    the plain feature (row-major upper triangle, sqrt(2) off the diagonal).
    """
    _check(np.asarray(x).shape[-1], g, kind)
    lifts = phi(_factors(x, g))                    # [..., g, P]
    if kind == "multi":
        return lifts.reshape(lifts.shape[:-2] + (-1,))
    return lifts.sum(axis=-2)


def factored_weights(q, k, g: int, kind: str) -> np.ndarray:
    """Attention weights from the factors' raw inner products.

    q [..., Tq, d], k [..., Tk, d] -> [..., Tq, Tk]: sum_a (q_a . k_a)^2 (multi)
    or sum_{a,b} (q_a . k_b)^2 (summed).
    """
    qf = _factors(q, g)                            # [..., Tq, g, p]
    kf = _factors(k, g)                            # [..., Tk, g, p]
    _check(qf.shape[-1] * g, g, kind)
    # dots[..., t, j, a, b] = q_{t,a} . k_{j,b}
    dots = np.einsum("...tap,...jbp->...tjab", qf, kf)
    if kind == "multi":
        return (np.diagonal(dots, axis1=-2, axis2=-1) ** 2).sum(-1)
    return (dots ** 2).sum(axis=(-2, -1))


def _prior(q_rows, g, kind, S0, z0):
    if S0 is None:
        return 0.0, 0.0
    fq = factored_phi(q_rows, g, kind)
    return fq @ S0, fq @ z0


def _rows(q_rows, t_idx, k, v, g, kind, causal, S0, z0):
    w = factored_weights(q_rows, k, g, kind)
    if causal:
        w = np.where(np.arange(k.shape[0])[None, :] <= t_idx[:, None], w, 0.0)
    pn, pd = _prior(q_rows, g, kind, S0, z0)
    return _safe_ratio(w @ v + pn, w.sum(axis=1) + pd)


def factored_brute_force(q, k, v, g: int, kind: str, causal: bool = True, S0=None, z0=None,
                         block: int = 512):
    """O(T^2) float64 definition [LA Definition; JA 2.1] with the factored weights.

    o_t = (sum_{j in J_t} w_tj v_j + phi(q_t).S0) / (sum_{j in J_t} w_tj + phi(q_t).z0),
    J_t = {0..t} (causal) or every token; (S0 [B,H,D,dv], z0 [B,H,D]) an optional
    initial state in the factored feature space. Rows in blocks of `block`.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    _check(d, g, kind)
    o = np.zeros((B, H, T, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, block):
                t1 = min(T, t0 + block)
                o[b, h, t0:t1] = _rows(q[b, h, t0:t1], np.arange(t0, t1), k[b, h], v[b, h], g,
                                       kind, causal,
                                       None if S0 is None else S0[b, h],
                                       None if z0 is None else z0[b, h])
    return o


def factored_brute_force_rows(q, k, v, rows, g: int, kind: str, causal: bool = True, S0=None,
                              z0=None):
    """Brute force for query positions `rows` only: [B, H, len(rows), dv]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    B, H = q.shape[:2]
    out = np.zeros((B, H, rows.size, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            out[b, h] = _rows(q[b, h, rows], rows, k[b, h], v[b, h], g, kind, causal,
                              None if S0 is None else S0[b, h],
                              None if z0 is None else z0[b, h])
    return out


def factored_recurrent(q, k, v, g: int, kind: str, S0=None, z0=None):
    """Token-by-token recurrence in the factored feature space [JA 1; LA]:
    S += phi(k_t) v_t^T, z += phi(k_t), then o_t = phi(q_t).S / phi(q_t).z.
    Returns (o, S_T [B,H,D,dv], z_T [B,H,D])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    D = factored_dim(d, g, kind)
    S = np.zeros((B, H, D, v.shape[-1])) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, D)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, H, T, v.shape[-1]))
    fq = factored_phi(q, g, kind)
    fk = factored_phi(k, g, kind)
    for t in range(T):
        S += fk[:, :, t, :, None] * v[:, :, t, None, :]
        z += fk[:, :, t]
        o[:, :, t] = _safe_ratio(np.einsum("bhp,bhpn->bhn", fq[:, :, t], S),
                                 np.einsum("bhp,bhp->bh", fq[:, :, t], z))
    return o, S, z


def factored_state_from_tokens(k, v, g: int, kind: str):
    """Total state of a token range: S = phi(K)^T V, z = phi(K)^T 1."""
    fk = factored_phi(k, g, kind)
    return np.einsum("bhtp,bhtn->bhpn", fk, np.asarray(v, np.float64)), fk.sum(axis=2)


def factored_chunked(q, k, v, C: int, g: int, kind: str, causal: bool = True, S0=None,
                     z0=None):
    """Exact chunked-state form [JA 2.3] with the factored feature.

    Chunk c covers [cC, min(cC + C, T)); its output takes the intra-chunk
    weights (from the factors' inner products, masked to j <= t) times [V | 1]
    plus phi(Q_c) times the exclusive prefix of chunk states (S0 first).
    Non-causal: one total state. Returns (o, S_T, z_T).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    D = factored_dim(d, g, kind)
    dv = v.shape[-1]
    if not causal:
        S, z = factored_state_from_tokens(k, v, g, kind)
        if S0 is not None:
            S, z = S + S0, z + z0
        fq = factored_phi(q, g, kind)
        return (_safe_ratio(np.einsum("bhtp,bhpn->bhtn", fq, S), np.einsum("bhtp,bhp->bht", fq, z)),
                S, z)
    S = np.zeros((B, H, D, dv)) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, D)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, H, T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Qc, Kc, Vc = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        n = Qc.shape[2]
        A = factored_weights(Qc, Kc, g, kind) * np.tril(np.ones((n, n)))
        fq = factored_phi(Qc, g, kind)
        num = A @ Vc + np.einsum("bhtp,bhpn->bhtn", fq, S)
        den = A.sum(axis=-1) + np.einsum("bhtp,bhp->bht", fq, z)
        o[:, :, sl] = _safe_ratio(num, den)
        Sc, zc = factored_state_from_tokens(Kc, Vc, g, kind)
        S, z = S + Sc, z + zc
    return o, S, z


def factored_decode_step(q, k, v, S, z, g: int, kind: str):
    """One recurrent step for N rows: q, k [N, d], v [N, dv], S [N, D, dv],
    z [N, D] -> (o, S + phi(k) v^T, z + phi(k)), o read after the update."""
    fk = factored_phi(k, g, kind)
    fq = factored_phi(q, g, kind)
    S2 = np.asarray(S, np.float64) + fk[:, :, None] * np.asarray(v, np.float64)[:, None, :]
    z2 = np.asarray(z, np.float64) + fk
    return (_safe_ratio(np.einsum("np,npv->nv", fq, S2), np.einsum("np,np->n", fq, z2)), S2, z2)
