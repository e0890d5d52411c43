"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the attention method: it only draws random
numbers (numpy PCG64, float64), shapes them into the workloads below and rounds
them to the kernel's input dtype with round-to-nearest-even. The oracle and the
GPU path both receive exactly the rounded values returned here.

Workloads (shapes and value distributions):

  tiny       B1 H1 T256    d_k16 d_v16 fp32 C64   q,k unit-norm Gaussian rows, v ~ N(0,1)
  fwd4k      B4 H8 T4096   d_k16 d_v64 bf16 C64   same distribution
  fwd32k     B1 H16 T32768 d_k32 d_v64 bf16 C128  same distribution
  fwd131k    B1 H8 T131072 d_k16 d_v64 bf16 C64   same distribution ("131k tokens")
  recall16k  B8 H4 T16384  d_k16 d_v64 bf16 C64   recall-shaped stream (below)
  decode     1024 steps on 512 sequences x 4 heads continuing recall16k

For the first-order (identity) feature, orthant_qkv draws the same shapes with
q, k on the nonnegative orthant (unit rows of |N(0, I)|), the cone on which that
feature's weights q.k are nonnegative. For the decay gate, log_decays draws
per-token log forget gates uniformly in [gmin, 0].

The recall-shaped stream stands in for the associative-recall and
repeated-key-overwrite workloads the pages evaluate on; no item of any public
suite is used. Per (b, h) stream: a codebook of 2048 unit Gaussian keys; at each
position t > 0, with probability 1/4 a key seen at a uniformly chosen earlier
position is re-bound to a new one-hot value different from its current one;
otherwise a key is drawn uniformly from the codebook, keeping its binding if it
has one and receiving a uniform one-hot value if not. The query at t is the key
of a uniformly chosen earlier position (q_0 = k_0).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "round_to", "gaussian_qkv", "orthant_qkv", "log_decays",
           "RecallStream",
           "recall_stream", "decode_continuation"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str        # "f32" or "bf16": input/output dtype of the kernel
    chunk: int
    seed: int
    tol: float        # max row-normwise relative error against float64
    kind: str = "gaussian"


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 256, 16, 16, "f32", 64, 1, 1e-4),
    "fwd4k": Workload("fwd4k", 4, 8, 4096, 16, 64, "bf16", 64, 2, 2e-2),
    "fwd32k": Workload("fwd32k", 1, 16, 32768, 32, 64, "bf16", 128, 3, 2e-2),
    "fwd131k": Workload("fwd131k", 1, 8, 131072, 16, 64, "bf16", 64, 4, 2e-2),
    "recall16k": Workload("recall16k", 8, 4, 16384, 16, 64, "bf16", 64, 5, 2e-2, "recall"),
}

DECODE_STEPS = 1024
DECODE_SEQS = 512


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to fp32 or bf16 (round-to-nearest-even), returned as
    float32 arrays that hold exactly representable values of that dtype."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    if dtype == "f32":
        return f
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype}")
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _unit_rows(rng, shape):
    g = rng.standard_normal(shape)
    return g / np.linalg.norm(g, axis=-1, keepdims=True)


def gaussian_qkv(B, H, T, dk, dv, seed, dtype="bf16"):
    """q, k: rows of N(0, I) normalised to unit L2 norm; v ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _unit_rows(rng, (B, H, T, dk))
    k = _unit_rows(rng, (B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def orthant_qkv(B, H, T, dk, dv, seed, dtype="bf16"):
    """q, k: rows of |N(0, I)| normalised to unit L2 norm (nonnegative); v ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = np.abs(_unit_rows(rng, (B, H, T, dk)))
    k = np.abs(_unit_rows(rng, (B, H, T, dk)))
    v = rng.standard_normal((B, H, T, dv))
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def log_decays(B, H, T, seed, gmin=-0.05):
    """Per-token log forget gates g ~ U(gmin, 0) (float32 [B,H,T]): the decay of
    the state at each token is exp(g) in (exp(gmin), 1]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(gmin, 0.0, (B, H, T)).astype(np.float32)


class RecallStream:
    """Vectorised generator of recall-shaped key/value/query streams.

    `n` independent streams advance together one position per call to `step`.
    Each stream owns a codebook of unit keys, a key -> value binding table and
    the codebook ids of its past keys.
    """

    def __init__(self, n, dk, dv, rng, capacity, codebook=2048, p_overwrite=0.25):
        self.n, self.dk, self.dv = n, dk, dv
        self.p = p_overwrite
        self.rng = rng
        self.codebook = _unit_rows(rng, (n, codebook, dk))
        self.cb_row = np.arange(n)
        self.binding = np.full((n, codebook), -1, dtype=np.int64)
        self.ar = np.arange(n)
        # past key ids: positions < base_len live in base[base_row], later ones in own
        self.base = np.zeros((n, 0), dtype=np.int32)
        self.base_row = self.ar
        self.base_len = 0
        self.own = np.zeros((n, capacity), dtype=np.int32)
        self.t = 0

    def continuation(self, index, rng, capacity):
        """New generator whose streams continue streams `index` of this one."""
        g = RecallStream.__new__(RecallStream)
        g.n, g.dk, g.dv, g.p, g.rng = len(index), self.dk, self.dv, self.p, rng
        g.codebook = self.codebook               # shared; row cb_row[i] serves stream i
        g.cb_row = self.cb_row[np.asarray(index)]
        g.binding = self.binding[index].copy()
        g.ar = np.arange(g.n)
        g.base = self.own[:, :self.t]
        g.base_row = np.asarray(index)
        g.base_len = self.t
        g.own = np.zeros((g.n, capacity), dtype=np.int32)
        g.t = self.t
        return g

    def _ids_at(self, j):
        jb = np.minimum(j, max(self.base_len - 1, 0))
        jo = np.maximum(j - self.base_len, 0)
        from_base = self.base[self.base_row, jb] if self.base_len else 0
        return np.where(j < self.base_len, from_base, self.own[self.ar, jo]).astype(np.int64)

    def step(self):
        """Advance one position; returns (query ids, key ids, value ids)."""
        rng, n, t = self.rng, self.n, self.t
        ncode = self.codebook.shape[1]
        fresh = rng.integers(0, ncode, size=n)
        if t > 0:
            earlier = self._ids_at(rng.integers(0, t, size=n))
            over = rng.random(n) < self.p
            key = np.where(over, earlier, fresh)
        else:
            over = np.zeros(n, dtype=bool)
            key = fresh
        cur = self.binding[self.ar, key]
        shift = rng.integers(1, self.dv, size=n)        # new value != current
        new_unbound = rng.integers(0, self.dv, size=n)
        val = np.where(over, (cur + shift) % self.dv, np.where(cur < 0, new_unbound, cur))
        self.binding[self.ar, key] = val
        qid = self._ids_at(rng.integers(0, t, size=n)) if t > 0 else key
        self.own[:, t - self.base_len] = key
        self.t += 1
        return qid, key, val

    def vectors(self, ids):
        return self.codebook[self.cb_row, ids]


def recall_stream(B, H, T, dk, dv, seed, dtype="bf16", return_gen=False):
    """Recall-shaped stream, [B, H, T, *] arrays (see the module docstring)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = RecallStream(B * H, dk, dv, rng, capacity=T)
    q = np.empty((B * H, T, dk))
    k = np.empty((B * H, T, dk))
    v = np.zeros((B * H, T, dv))
    for t in range(T):
        qid, kid, vid = gen.step()
        q[:, t] = gen.vectors(qid)
        k[:, t] = gen.vectors(kid)
        v[gen.ar, t, vid] = 1.0
    out = tuple(round_to(a.reshape(B, H, T, -1), dtype) for a in (q, k, v))
    return (out + (gen,)) if return_gen else out


def decode_continuation(gen: RecallStream, H, n_seq, steps, seed, dtype="bf16"):
    """Decode tokens for n_seq sequences x H heads continuing a recall stream
    generator built over B*H streams. Sequence s continues stream b = s mod B, so
    each (b, h) stream is replicated n_seq / B times; all continuations draw from
    one PCG64 generator seeded with `seed`.

    Returns q, k [steps, n_seq, H, dk], v [steps, n_seq, H, dv] and the source
    stream index (b*H + h) of every (sequence, head) row, shape [n_seq*H].
    """
    B = gen.n // H
    src = np.array([(s % B) * H + h for s in range(n_seq) for h in range(H)])
    g = gen.continuation(src, np.random.Generator(np.random.PCG64(seed)), capacity=steps)
    N = n_seq * H
    q = np.empty((steps, N, gen.dk))
    k = np.empty((steps, N, gen.dk))
    v = np.zeros((steps, N, gen.dv))
    for t in range(steps):
        qid, kid, vid = g.step()
        q[t] = g.vectors(qid)
        k[t] = g.vectors(kid)
        v[t, g.ar, vid] = 1.0
    shape = (steps, n_seq, H)
    return (round_to(q.reshape(shape + (-1,)), dtype), round_to(k.reshape(shape + (-1,)), dtype),
            round_to(v.reshape(shape + (-1,)), dtype), src)
