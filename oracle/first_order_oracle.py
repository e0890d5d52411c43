"""Plain float64 CPU oracle for first-order kernelized linear attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or call this module. The library (the HIP path behind
the C ABI) never does, and this module imports nothing from the library.

Sources (web pages describing arXiv 2607.17419, "Kernelized Linear Attention:
Breaking the Capacity Wall with Symmetric Cones"):

  [ABS]  the paper's English abstract (fugumt.com summary page): an associative
         scan of the first-order feature is set against a matched sequential
         linear-attention baseline
  [JA]   gist.science Japanese explainer, technical summary 2.2 (orthant, the
         cone of the first-order feature) and 2.3 (chunk parallelism, recurrence
         depth O(N_C) sequential versus O(log N_C) with a scan)
  [LA]   notes.yuuk.io wiki page on linear attention, "Definition"

What is computed (restated, not quoted): the first-order feature is the
identity, phi1(x) = x, so the attention weight is the raw inner product
w_tj = q_t . k_j and the state is S = sum_j k_j v_j^T (d x d_v) with
z = sum_j k_j. The output is the same normalised form as for the PSD lift:
o_t = sum_{j<=t} w_tj v_j / sum_{j<=t} w_tj, zero where the denominator is 0.

Readings (listed in the design notes): the pages do not print the baseline's
formula. The normalised form above is taken so that the two features differ
only in phi; it is a convex gate when the weights are nonnegative, which the
orthant cone of [JA 2.2] gives for nonnegative queries and keys. Nothing else
(no epsilon, no temperature) is added; a zero denominator gives a zero output,
as for the PSD lift.

Parity pins: tests/first_order_checks.py. None of these functions is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = ["fo_brute_force", "fo_recurrent", "fo_state_from_tokens", "fo_chunked"]


def _safe_ratio(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """num / den, and 0 where den == 0."""
    den_b = den[..., None]
    out = np.zeros(np.broadcast_shapes(num.shape, den_b.shape), dtype=np.float64)
    nz = np.broadcast_to(den_b != 0.0, out.shape)
    np.divide(num, den_b, out=out, where=nz)
    return out


# ---------------------------------------------------------------------------
# Plain definition  [LA Definition with phi1(x) = x]
# ---------------------------------------------------------------------------

def fo_brute_force(q, k, v, causal: bool = True, S0=None, z0=None):
    """O(T^2) float64 reference for every (b, h, t): w_tj = q_t . k_j and
    o_t = sum_{j in J_t} w_tj v_j / sum_{j in J_t} w_tj, J_t = {0..t} (causal)
    or every token. An optional initial state S0 [B,H,d,dv], z0 [B,H,d] stands
    for earlier tokens and adds q_t.S0 and q_t.z0."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, _ = q.shape
    o = np.zeros((B, H, T, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            w = q[b, h] @ k[b, h].T                     # [T query, T key]
            if causal:
                w = w * np.tril(np.ones((T, T)))         # j <= t
            num = w @ v[b, h]
            den = w.sum(axis=1)
            if S0 is not None:
                num = num + q[b, h] @ np.asarray(S0[b, h], np.float64)
                den = den + q[b, h] @ np.asarray(z0[b, h], np.float64)
            o[b, h] = _safe_ratio(num, den)
    return o


# ---------------------------------------------------------------------------
# Recurrent form  [ABS, LA: a fixed-size state updated token by token]
# ---------------------------------------------------------------------------

def fo_recurrent(q, k, v, S0=None, z0=None):
    """S += k_t v_t^T, z += k_t, then o_t = q_t.S / q_t.z (token t included).
    Returns (o [B,H,T,dv], S_T [B,H,d,dv], z_T [B,H,d])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, d, dv)) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, d)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        S += k[:, :, t, :, None] * v[:, :, t, None, :]
        z += k[:, :, t, :]
        num = np.einsum("bha,bhan->bhn", q[:, :, t], S)
        den = np.einsum("bha,bha->bh", q[:, :, t], z)
        o[:, :, t] = _safe_ratio(num, den)
    return o, S, z


def fo_state_from_tokens(k, v):
    """State of a token range: S = K^T V [B,H,d,dv], z = K^T 1 [B,H,d]."""
    k = np.asarray(k, np.float64)
    S = np.einsum("bhta,bhtn->bhan", k, np.asarray(v, np.float64))
    return S, k.sum(axis=2)


# ---------------------------------------------------------------------------
# Chunked-state form  [JA 2.3: intra-chunk term plus the state of earlier chunks]
# ---------------------------------------------------------------------------

def fo_chunked(q, k, v, C: int, causal: bool = True, S0=None, z0=None):
    """Chunk c = tokens [cC, min(cC+C, T)): num = A V_c + Q_c P_c and
    den = A 1 + Q_c Z_c with A = Q_c K_c^T masked to j <= t, (P_c, Z_c) the
    state of every earlier chunk (plus S0, z0), walked chunk by chunk.
    Non-causal: one state over every token. Returns (o, S_T, z_T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, d, dv)) if S0 is None else np.array(S0, np.float64)
    z = np.zeros((B, H, d)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, H, T, dv))
    if not causal:
        St, zt = fo_state_from_tokens(k, v)
        S, z = S + St, z + zt
        num = np.einsum("bhta,bhan->bhtn", q, S)
        den = np.einsum("bhta,bha->bht", q, z)
        return _safe_ratio(num, den), S, z
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Qc, Kc, Vc = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        n = Qc.shape[2]
        A = np.einsum("bhta,bhja->bhtj", Qc, Kc) * np.tril(np.ones((n, n)))
        num = np.einsum("bhtj,bhjn->bhtn", A, Vc) + np.einsum("bhta,bhan->bhtn", Qc, S)
        den = A.sum(axis=-1) + np.einsum("bhta,bha->bht", Qc, z)
        o[:, :, sl] = _safe_ratio(num, den)
        Sc, zc = fo_state_from_tokens(Kc, Vc)
        S, z = S + Sc, z + zc
    return o, S, z
