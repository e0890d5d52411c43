"""Plain float64 CPU oracle for DeltaKATA, the delta-rule variant of KATA.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or call this module. The library (the HIP path behind
the C ABI) never does, and this module imports nothing from the library.

Sources (web pages describing arXiv 2607.17419, "Kernelized Linear Attention:
Breaking the Capacity Wall with Symmetric Cones"):

  [JA]   gist.science Japanese explainer: technical summary 1 (gated linear
         RNNs such as DeltaNet and Gated DeltaNet, which erase by content),
         2.1 (the normalised output gate), 2.3 (the chunked-state form) and 4
         (repeated-key overwrite: the delta-rule variant, DeltaKATA, corrects
         stale bindings at repeated addresses)
  [IT]   gist.science Italian explainer, the same sections
  [ABS]  the paper's abstract: delta rules are among the mechanisms whose
         interaction with the feature geometry the paper studies

The pages print no formula for DeltaKATA. Reading taken (listed in the design
notes): the delta rule of DeltaNet applied to the KATA state. With the lifted
key scaled to unit norm, kappa_t = phi(k_t) / |k_t|^2 (|phi(k)| = |k|^2 for the
packed lift; kappa = 0 for k = 0), and a write strength beta_t in [0, 1] per
token and head, the numerator state S and the denominator state z form one
augmented state A = [S | z] whose value for token t is u_t = [v_t, 1]:

    A_t = A_{t-1} + beta_t kappa_t (u_t - kappa_t^T A_{t-1}),
    o_t = phi(q_t).S_t / phi(q_t).z_t        (0 where the denominator is 0),

so the readout keeps KATA's normalised form and reads the state after token t
(as the plain forward does). beta = 0 leaves the state unchanged; beta = 1
makes kappa_t^T A_t = u_t, i.e. the state returns exactly the latest value for
that key (the overwrite of [JA 4]); with mutually orthogonal unit keys the erase
term vanishes and beta = 1 gives plain KATA.

The chunked form restates the delta rule's chunk recursion over the pages'
chunked-state structure [JA 2.3]: inside a chunk of keys K (rows kappa_t) the
pseudo-values P = beta (U - K A_prev) minus the corrections of earlier tokens of
the chunk solve a unit lower-triangular system, the outputs read the state
before the chunk plus the chunk's own tokens through the inclusive causal mask,
and the state gains K^T P. A library linear solve serves as a step.

Parity pins: tests/delta_checks.py (run by tests/test_delta_oracle.py with a
planted-mistake suite). None of these functions is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .kata_oracle import _safe_ratio, phi, phi_dim

__all__ = ["delta_kappa", "delta_recurrent", "delta_chunked", "delta_decode_step"]


def delta_kappa(k):
    """Unit-norm lifted keys phi(k) / |k|^2 of the last axis (0 for k = 0)."""
    k = np.asarray(k, np.float64)
    n2 = (k * k).sum(-1, keepdims=True)
    out = np.zeros(k.shape[:-1] + (phi_dim(k.shape[-1]),))
    np.divide(phi(k), n2, out=out, where=n2 != 0.0)
    return out


def _aug(S0, z0, B, H, D, dv):
    A = np.zeros((B, H, D, dv + 1))
    if S0 is not None:
        A[..., :dv] = S0
        A[..., dv] = z0
    return A


def delta_recurrent(q, k, v, beta, S0=None, z0=None, parts=False):
    """Token-by-token DeltaKATA. q, k [B,H,T,d], v [B,H,T,dv], beta [B,H,T].
    Returns (o [B,H,T,dv], S [B,H,D,dv], z [B,H,D]), the state after the last
    token; with parts=True, (num [B,H,T,dv], den [B,H,T], S, z) instead, the
    readout's numerator and denominator before the division."""
    q = np.asarray(q, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    D = phi_dim(d)
    A = _aug(S0, z0, B, H, D, dv)
    kap = delta_kappa(k)
    fq = phi(q)
    o = np.zeros((B, H, T, dv))
    num = np.zeros((B, H, T, dv))
    den = np.zeros((B, H, T))
    for t in range(T):
        u = np.concatenate([v[:, :, t], np.ones((B, H, 1))], -1)          # [B,H,dv+1]
        kt = kap[:, :, t]                                                   # [B,H,D]
        erase = np.einsum("bhp,bhpc->bhc", kt, A)                          # kappa^T A
        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]
        r = np.einsum("bhp,bhpc->bhc", fq[:, :, t], A)
        o[:, :, t] = _safe_ratio(r[..., :dv], r[..., dv])
        num[:, :, t] = r[..., :dv]
        den[:, :, t] = r[..., dv]
    if parts:
        return num, den, A[..., :dv], A[..., dv]
    return o, A[..., :dv], A[..., dv]


def delta_chunked(q, k, v, beta, C: int, S0=None, z0=None):
    """The same outputs and final state through chunks of C tokens (the last
    chunk ragged): for chunk c with unit keys K [n, D], values U = [V, 1] and
    strengths b, the pseudo-values P solve (I + diag(b) L) P = diag(b)(U - K A),
    L the strictly lower part of K K^T; the outputs are
    phi(Q) A + mask(phi(Q) K^T) P with the inclusive causal mask; then
    A += K^T P."""
    q = np.asarray(q, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    D = phi_dim(d)
    A = _aug(S0, z0, B, H, D, dv)
    kap = delta_kappa(k)
    fq = phi(q)
    o = np.zeros((B, H, T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        K = kap[:, :, c0:c1]                                               # [B,H,n,D]
        U = np.concatenate([v[:, :, c0:c1], np.ones((B, H, n, 1))], -1)   # [B,H,n,dv+1]
        b = beta[:, :, c0:c1]
        L = np.tril(K @ np.swapaxes(K, -1, -2), -1)
        M = np.eye(n) + b[..., :, None] * L
        rhs = b[..., :, None] * (U - K @ A)
        P = np.linalg.solve(M, rhs)
        Q = fq[:, :, c0:c1]
        W = np.tril(Q @ np.swapaxes(K, -1, -2))                            # j <= t
        r = Q @ A + W @ P
        o[:, :, c0:c1] = _safe_ratio(r[..., :dv], r[..., dv])
        A = A + np.swapaxes(K, -1, -2) @ P
    return o, A[..., :dv], A[..., dv]


def delta_decode_step(q, k, v, beta, S, z):
    """One recurrent step on rows [N, d] from the state (S [N,D,dv], z [N,D]):
    returns (o [N,dv], S, z) after the update."""
    o, S1, z1 = delta_recurrent(np.asarray(q)[None, :, None], np.asarray(k)[None, :, None],
                                np.asarray(v)[None, :, None],
                                np.asarray(beta, np.float64).reshape(1, -1, 1),
                                np.asarray(S, np.float64)[None], np.asarray(z, np.float64)[None])
    return o[0, :, 0], S1[0], z1[0]
