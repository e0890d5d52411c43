"""Plain float64 CPU oracle for the decay-gated KATA forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or call this module. The library (the HIP path behind
the C ABI) never does, and this module imports nothing from the library.

Sources (web pages describing arXiv 2607.17419, "Kernelized Linear Attention:
Breaking the Capacity Wall with Symmetric Cones"):

  [ABS]  the paper's abstract (fugumt.com summary page): decay gates are among
         the mechanisms whose interaction with the feature geometry the paper
         studies; the recurrence keeps a fixed-size state
  [JA]   gist.science Japanese explainer, technical summary 1 (gated linear RNNs
         with learned forget gates), 2.1 (the normalised output gate) and 2.3
         (chunked state with an associative scan over chunk states)

The pages print no decay formula. Reading taken (listed in the design notes):
a scalar forget gate per token and head, given as its logarithm g_t <= 0
(gamma_t = exp(g_t) in (0, 1]), that scales the whole state before token t is
added:

    S_t = gamma_t S_{t-1} + phi(k_t) v_t^T,   z_t = gamma_t z_{t-1} + phi(k_t),
    o_t = phi(q_t).S_t / phi(q_t).z_t   (0 where the denominator is 0),

with S_{-1} = S0, z_{-1} = z0. Unrolled, the weight of key j for query t is
(q_t . k_j)^2 exp(G_t - G_j) with G the inclusive cumulative sum of g, so the
weights stay nonnegative and the output stays a convex combination; the initial
state enters with factor exp(G_t). In the chunked form a chunk's state is paired
with its total decay a = exp(sum of its g), and chunk states combine with the
associative, non-commutative operator

    (a1, S1) o (a2, S2) = (a1 a2, a2 S1 + S2)      (1 earlier, 2 later).

Every function also takes feature="identity" for the first-order feature
phi1(x) = x of the first-order oracle (oracle/first_order_oracle.py): the
weight of key j for query t is then (q_t . k_j) exp(G_t - G_j) and the state
is d x d_v; the gate acts the same way.

Parity pins: tests/decay_checks.py. None of these functions is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

from .kata_oracle import _safe_ratio, phi, phi_dim

__all__ = ["decay_brute_force", "decay_brute_force_rows", "decay_recurrent", "decay_combine",
           "decay_prefix_states", "decay_chunked", "decay_decode_step"]


def _cum(g):
    return np.cumsum(np.asarray(g, np.float64), axis=-1)


def _lift(x, feature):
    """The feature map: the PSD lift phi, or the identity."""
    if feature == "psd":
        return phi(x)
    if feature == "identity":
        return np.asarray(x, np.float64)
    raise ValueError(feature)


def _weight(s, feature):
    """phi(q).phi(k) from s = q.k: s^2 for the PSD lift, s for the identity."""
    return s ** 2 if feature == "psd" else s


def _dim(d, feature):
    return phi_dim(d) if feature == "psd" else d


# ---------------------------------------------------------------------------
# Plain definition: weights (q_t . k_j)^2 exp(G_t - G_j), j <= t
# ---------------------------------------------------------------------------

def decay_brute_force(q, k, v, g, S0=None, z0=None, feature="psd"):
    """O(T^2) float64 reference. g [B,H,T] log-decays (<= 0)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    G = _cum(g)
    B, H, T, _ = q.shape
    o = np.zeros((B, H, T, v.shape[-1]))
    t_idx = np.arange(T)
    mask = t_idx[None, :] <= t_idx[:, None]
    for b in range(B):
        for h in range(H):
            diff = np.where(mask, G[b, h][:, None] - G[b, h][None, :], -np.inf)
            w = _weight(q[b, h] @ k[b, h].T, feature) * np.exp(diff)
            num = w @ v[b, h]
            den = w.sum(axis=1)
            if S0 is not None:
                e = np.exp(G[b, h])[:, None]
                fq = _lift(q[b, h], feature)
                num = num + e * (fq @ np.asarray(S0[b, h], np.float64))
                den = den + e[:, 0] * (fq @ np.asarray(z0[b, h], np.float64))
            o[b, h] = _safe_ratio(num, den)
    return o


def decay_brute_force_rows(q, k, v, g, rows, feature="psd"):
    """The same definition for the query positions `rows` only (every b, h):
    O(T) per row, for spot checks of long sequences. Returns [B,H,len(rows),dv]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    G = _cum(g)
    B, H, T, _ = q.shape
    o = np.zeros((B, H, len(rows), v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for i, t in enumerate(rows):
                w = _weight(k[b, h, :t + 1] @ q[b, h, t], feature) * np.exp(G[b, h, t] - G[b, h, :t + 1])
                den = w.sum()
                o[b, h, i] = (w @ v[b, h, :t + 1]) / den if den != 0.0 else 0.0
    return o


# ---------------------------------------------------------------------------
# Recurrent form: decay the state, add the token, read
# ---------------------------------------------------------------------------

def decay_recurrent(q, k, v, g, S0=None, z0=None, feature="psd"):
    """Returns (o [B,H,T,dv], S_T [B,H,D,dv], z_T [B,H,D])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    D = _dim(d, feature)
    S = np.zeros((B, H, D, dv)) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, D)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, H, T, dv))
    fq, fk = _lift(q, feature), _lift(k, feature)
    for t in range(T):
        gam = np.exp(g[:, :, t])
        S = gam[:, :, None, None] * S + fk[:, :, t, :, None] * v[:, :, t, None, :]
        z = gam[:, :, None] * z + fk[:, :, t, :]
        num = np.einsum("bhp,bhpn->bhn", fq[:, :, t], S)
        den = np.einsum("bhp,bhp->bh", fq[:, :, t], z)
        o[:, :, t] = _safe_ratio(num, den)
    return o, S, z


def decay_decode_step(q, k, v, g, S, z, feature="psd"):
    """One decode step for N rows: q, k [N,d], v [N,dv], g [N], S [N,D,dv],
    z [N,D]. Returns (o, S', z') with S' = exp(g) S + phi(k) v^T."""
    gam = np.exp(np.asarray(g, np.float64))
    fk = _lift(k, feature)
    fq = _lift(q, feature)
    S2 = gam[:, None, None] * np.asarray(S, np.float64) + fk[:, :, None] * np.asarray(v, np.float64)[:, None, :]
    z2 = gam[:, None] * np.asarray(z, np.float64) + fk
    num = np.einsum("np,npv->nv", fq, S2)
    den = np.einsum("np,np->n", fq, z2)
    return _safe_ratio(num, den), S2, z2


# ---------------------------------------------------------------------------
# Chunked form with the decay-aware scan  [JA 2.3 with the gate above]
# ---------------------------------------------------------------------------

def decay_combine(x, y):
    """(a1, S1, z1) o (a2, S2, z2) = (a1 a2, a2 S1 + S2, a2 z1 + z2): the state
    after the span of x followed by the span of y (a: [B,H])."""
    a1, S1, z1 = x
    a2, S2, z2 = y
    return a1 * a2, a2[..., None, None] * S1 + S2, a2[..., None] * z1 + z2


def _chunk_state(k, v, g, feature):
    """(a, S, z) of one span: a = exp(sum g), S = sum_j exp(G_last - G_j) phi(k_j) v_j^T."""
    G = _cum(g)
    wgt = np.exp(G[..., -1:] - G)                              # [B,H,n]
    fk = _lift(k, feature) * wgt[..., None]
    S = np.einsum("bhtp,bhtn->bhpn", fk, np.asarray(v, np.float64))
    return np.exp(G[..., -1]), S, fk.sum(axis=2)


def decay_prefix_states(k, v, g, C: int, S0=None, z0=None, feature="psd"):
    """Exclusive prefixes (P_c, Z_c) of the chunk states under decay_combine,
    computed by a Hillis-Steele (log-depth) inclusive scan over chunks, shifted
    by one and started from (S0, z0). Returns (P [B,H,NC,D,dv], Z [B,H,NC,D],
    S_T, z_T)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    B, H, T, d = k.shape
    dv = v.shape[-1]
    D = _dim(d, feature)
    NC = -(-T // C)
    items = [_chunk_state(k[:, :, c * C:(c + 1) * C], v[:, :, c * C:(c + 1) * C],
                          g[:, :, c * C:(c + 1) * C], feature) for c in range(NC)]
    init = (np.ones((B, H)), np.zeros((B, H, D, dv)) if S0 is None else np.array(S0, np.float64),
            np.zeros((B, H, D)) if z0 is None else np.array(z0, np.float64))
    seq = [init] + items                                      # exclusive: identity-like start
    step = 1
    while step < len(seq):                                    # inclusive scan, log depth
        seq = [seq[i] if i < step else decay_combine(seq[i - step], seq[i]) for i in range(len(seq))]
        step *= 2
    P = np.stack([seq[c][1] for c in range(NC)], axis=2)
    Z = np.stack([seq[c][2] for c in range(NC)], axis=2)
    return P, Z, seq[NC][1], seq[NC][2]


def decay_chunked(q, k, v, g, C: int, S0=None, z0=None, feature="psd"):
    """Chunk c: num = A V_c + exp(b_t) phi(Q_c) P_c, den = A 1 + exp(b_t) phi(Q_c) Z_c,
    A_tj = (q_t . k_j)^2 exp(b_t - b_j) masked to j <= t (q_t . k_j for the
    identity), b the cumulative log-decay inside the chunk. Returns (o, S_T, z_T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    B, H, T, d = q.shape
    o = np.zeros((B, H, T, v.shape[-1]))
    P, Z, S_T, z_T = decay_prefix_states(k, v, g, C, S0, z0, feature)
    for c in range(P.shape[2]):
        sl = slice(c * C, min(T, (c + 1) * C))
        Qc, Kc, Vc = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        b = _cum(g[:, :, sl])
        n = Qc.shape[2]
        tri = np.tril(np.ones((n, n), dtype=bool))
        diff = np.where(tri, b[..., :, None] - b[..., None, :], -np.inf)
        A = _weight(np.einsum("bhtd,bhjd->bhtj", Qc, Kc), feature) * np.exp(diff)
        e = np.exp(b)
        fq = _lift(Qc, feature)
        num = np.einsum("bhtj,bhjn->bhtn", A, Vc) + e[..., None] * np.einsum("bhtp,bhpn->bhtn", fq, P[:, :, c])
        den = A.sum(axis=-1) + e * np.einsum("bhtp,bhp->bht", fq, Z[:, :, c])
        o[:, :, sl] = _safe_ratio(num, den)
    return o, S_T, z_T
