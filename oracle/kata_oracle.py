"""Plain float64 CPU oracle for the KATA causal forward (rank-one PSD feature).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or call this module. The library (the HIP path behind
the C ABI) never does, and this module imports nothing from the library.

Sources (web pages describing arXiv 2607.17419, "Kernelized Linear Attention:
Breaking the Capacity Wall with Symmetric Cones"):

  [ABS]   the paper's English abstract, as shown on the fugumt.com summary page
  [JA]    gist.science Japanese explainer, technical summary, sections 1, 2.1,
          2.2, 2.3 and 4
  [IT]    gist.science Italian explainer, the same sections
  [LA]    notes.yuuk.io wiki page on linear attention (線形注意), "Definition"

What the method computes (restated, not quoted):

* Feature map [JA 2.2, IT 2.2, ABS]: the rank-one PSD lift psi(u) = u u^T. The
  Frobenius inner product of two lifts is the square of the raw inner product,
  so every attention weight is nonnegative.
* Attention [LA Definition; JA 2.1; ABS]: normalised kernelised linear
  attention o_t = phi(q_t)^T S_t / phi(q_t)^T z_t with S_t = sum_j phi(k_j) v_j^T
  and z_t = sum_j phi(k_j). The denominator is the parameter-free convex output
  gate of [JA 2.1] / [ABS], which blends the previous readout with the current
  value, so the sum runs over j <= t (token t included).
* Forms of the computation: recurrent with a fixed-size state [JA 1; ABS; LA];
  exact O(T) chunked-state form with an associative scan over chunk states
  [JA 2.3; IT 2.3; ABS].

Readings where the pages are silent (each is listed in the design notes):

* Packing: the d(d+1)/2 unique entries of x x^T in row-major upper-triangle
  order p(i, j) = i*d - i*(i-1)/2 + (j - i), i <= j; diagonal entries x_i^2,
  off-diagonal entries sqrt(2) x_i x_j, so that phi(q).phi(k) = (q.k)^2.
* No temperature and no epsilon; a zero denominator gives a zero output.
* Ragged last chunk: chunk c covers tokens [cC, min(cC + C, T)).
* Non-causal mode sums over every token.

Parity pins (tests/test_oracle_pins.py) tie every function here to closed forms,
invariants and brute force on tiny inputs; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "phi_dim", "pack_pairs", "phi", "brute_force", "brute_force_rows",
    "recurrent", "chunked", "prefix_states", "decode_step", "state_from_tokens",
]

SQRT2 = math.sqrt(2.0)


# ---------------------------------------------------------------------------
# Feature map  [JA 2.2 / IT 2.2: psi(u) = u u^T squares the inner product]
# ---------------------------------------------------------------------------

def phi_dim(d: int) -> int:
    """Number of unique entries of a symmetric d x d matrix, d(d+1)/2."""
    return d * (d + 1) // 2


def pack_pairs(d: int) -> list[tuple[int, int]]:
    """(i, j), i <= j, in packing order: row-major over the upper triangle."""
    return [(i, j) for i in range(d) for j in range(i, d)]


def phi(x: np.ndarray) -> np.ndarray:
    """Packed rank-one PSD feature of the last axis: x [..., d] -> [..., D].

    Entry p(i, j) holds x_i x_j on the diagonal and sqrt(2) x_i x_j off it, so
    the Euclidean dot product of two packed vectors equals the Frobenius
    product of the two lifts x x^T, i.e. the squared raw inner product.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    out = np.empty(x.shape[:-1] + (phi_dim(d),), dtype=np.float64)
    for p, (i, j) in enumerate(pack_pairs(d)):
        scale = 1.0 if i == j else SQRT2
        out[..., p] = scale * x[..., i] * x[..., j]
    return out


def _safe_ratio(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """num / den with the zero-denominator rule: o = 0 where den == 0."""
    den_b = den[..., None]
    out = np.zeros(np.broadcast_shapes(num.shape, den_b.shape), dtype=np.float64)
    nz = np.broadcast_to(den_b != 0.0, out.shape)
    np.divide(num, den_b, out=out, where=nz)
    return out


def _prior(q_rows, S0, z0):
    """Contribution of an initial state (tokens before this call) to num, den."""
    if S0 is None:
        return 0.0, 0.0
    fq = phi(q_rows)
    return fq @ S0, fq @ z0


# ---------------------------------------------------------------------------
# Brute force: the plain definition  [LA Definition; JA 2.1; ABS]
# ---------------------------------------------------------------------------

def brute_force(q, k, v, causal: bool = True, S0=None, z0=None, block: int = 512):
    """O(T^2) float64 reference for every (b, h, t).

    w_tj = (q_t . k_j)^2, o_t = sum_{j in J_t} w_tj v_j / sum_{j in J_t} w_tj with
    J_t = {0..t} (causal) or {0..T-1}. An optional initial state (S0 [B,H,D,dv],
    z0 [B,H,D]) stands for earlier tokens and adds phi(q_t).S0 and phi(q_t).z0.
    Rows are processed in blocks of `block` queries to bound memory; that is the
    only restructuring.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, block):
                t1 = min(T, t0 + block)
                o[b, h, t0:t1] = _rows(q[b, h, t0:t1], np.arange(t0, t1), k[b, h], v[b, h],
                                       causal,
                                       None if S0 is None else S0[b, h],
                                       None if z0 is None else z0[b, h])
    return o


def _rows(q_rows, t_idx, k, v, causal, S0, z0):
    w = (q_rows @ k.T) ** 2                       # (q_t . k_j)^2, nonnegative
    if causal:
        w = np.where(np.arange(k.shape[0])[None, :] <= t_idx[:, None], w, 0.0)
    num = w @ v
    den = w.sum(axis=1)
    pn, pd = _prior(q_rows, S0, z0)
    return _safe_ratio(num + pn, den + pd)


def brute_force_rows(q, k, v, rows, causal: bool = True, S0=None, z0=None):
    """Brute force for a subset of query positions `rows` (same for all b, h).

    Returns [B, H, len(rows), dv]. Used for sampled parity at full sizes.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    B, H = q.shape[:2]
    out = np.zeros((B, H, rows.size, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = _rows(q[b, h, rows], rows, k[b, h], v[b, h], causal,
                              None if S0 is None else S0[b, h],
                              None if z0 is None else z0[b, h])
    return out


# ---------------------------------------------------------------------------
# Recurrent form  [JA 1, ABS: constant-time recurrence with a fixed state; LA]
# ---------------------------------------------------------------------------

def recurrent(q, k, v, S0=None, z0=None):
    """Token-by-token recurrence: S += phi(k_t) v_t^T, z += phi(k_t), then read
    o_t = phi(q_t).S / phi(q_t).z (update first: token t is included).

    Returns (o [B,H,T,dv], S_T [B,H,D,dv], z_T [B,H,D]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    D = phi_dim(d)
    S = np.zeros((B, H, D, dv)) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, D)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, H, T, dv))
    fq = phi(q)
    fk = phi(k)
    for t in range(T):
        S += fk[:, :, t, :, None] * v[:, :, t, None, :]
        z += fk[:, :, t, :]
        num = np.einsum("bhp,bhpn->bhn", fq[:, :, t], S)
        den = np.einsum("bhp,bhp->bh", fq[:, :, t], z)
        o[:, :, t] = _safe_ratio(num, den)
    return o, S, z


def decode_step(q, k, v, S, z):
    """One recurrent decode step for N independent (sequence, head) rows.

    q, k [N, d]; v [N, dv]; S [N, D, dv]; z [N, D]. Returns (o, S', z') with
    S' = S + phi(k) v^T, z' = z + phi(k), o = phi(q).S' / phi(q).z'.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    fk = phi(k)
    fq = phi(q)
    S2 = np.asarray(S, np.float64) + fk[:, :, None] * v[:, None, :]
    z2 = np.asarray(z, np.float64) + fk
    num = np.einsum("np,npv->nv", fq, S2)
    den = np.einsum("np,np->n", fq, z2)
    return _safe_ratio(num, den), S2, z2


def state_from_tokens(k, v):
    """Total state of a token range: S = phi(K)^T V, z = phi(K)^T 1."""
    fk = phi(k)
    S = np.einsum("bhtp,bhtn->bhpn", fk, np.asarray(v, np.float64))
    return S, fk.sum(axis=2)


# ---------------------------------------------------------------------------
# Exact chunked-state form  [JA 2.3, IT 2.3, ABS: intra-chunk term + inter-chunk
# state propagated by a prefix over chunk states]
# ---------------------------------------------------------------------------

def prefix_states(k, v, C: int, S0=None, z0=None):
    """Exclusive prefix of per-chunk states.

    Chunk c covers tokens [cC, min(cC+C, T)). Its state is S_c = phi(K_c)^T V_c,
    z_c = phi(K_c)^T 1. The prefix is P_c = S0 + sum_{c' < c} S_{c'} (likewise
    Z_c); the scan operator is elementwise addition with identity 0 (or S0).
    Returns (P [B,H,NC,D,dv], Z [B,H,NC,D], S_T, z_T).
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = k.shape
    dv = v.shape[-1]
    D = phi_dim(d)
    NC = -(-T // C)
    P = np.zeros((B, H, NC, D, dv))
    Z = np.zeros((B, H, NC, D))
    S = np.zeros((B, H, D, dv)) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, D)) if z0 is None else np.array(z0, np.float64)
    for c in range(NC):
        P[:, :, c] = S
        Z[:, :, c] = z
        Sc, zc = state_from_tokens(k[:, :, c * C:(c + 1) * C], v[:, :, c * C:(c + 1) * C])
        S = S + Sc
        z = z + zc
    return P, Z, S, z


def chunked(q, k, v, C: int, causal: bool = True, S0=None, z0=None):
    """Exact chunked-state forward in float64.

    Causal: for chunk c, num = A V_c + phi(Q_c) P_c and den = A 1 + phi(Q_c) Z_c,
    where A = (Q_c K_c^T)^2 masked to j <= t inside the chunk and (P_c, Z_c) is
    the exclusive prefix of chunk states. Non-causal: one global state.
    Returns (o, S_T, z_T).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    if not causal:
        S, z = state_from_tokens(k, v)
        if S0 is not None:
            S = S + S0
            z = z + z0
        fq = phi(q)
        o = _safe_ratio(np.einsum("bhtp,bhpn->bhtn", fq, S), np.einsum("bhtp,bhp->bht", fq, z))
        return o, S, z
    P, Z, S_T, z_T = prefix_states(k, v, C, S0, z0)
    for c in range(P.shape[2]):
        sl = slice(c * C, min(T, (c + 1) * C))
        Qc, Kc, Vc = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        n = Qc.shape[2]
        A = np.einsum("bhtd,bhjd->bhtj", Qc, Kc) ** 2
        A = A * np.tril(np.ones((n, n)))                      # j <= t inside the chunk
        fq = phi(Qc)
        num = np.einsum("bhtj,bhjn->bhtn", A, Vc) + np.einsum("bhtp,bhpn->bhtn", fq, P[:, :, c])
        den = A.sum(axis=-1) + np.einsum("bhtp,bhp->bht", fq, Z[:, :, c])
        o[:, :, sl] = _safe_ratio(num, den)
    return o, S_T, z_T
