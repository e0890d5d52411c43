"""Helpers for the GPU parity tests: device transfer, error norms, input cache."""
from __future__ import annotations

import functools
import sys

import numpy as np

from kernelized_linear_attention_phi_amd import inputs as gen


def say(msg):
    """Flush a progress line (names the case before each GPU step)."""
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def dev(a, dtype="f32"):
    """float32 numpy array holding exact values of `dtype` -> GPU tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(torch_dtype(dtype))


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def row_rel_err(got, ref):
    """max over rows of |got - ref|_inf / |ref|_inf; rows whose reference is all
    zero must be exactly zero (returned error inf otherwise)."""
    got = np.asarray(got, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    scale = np.abs(ref).max(axis=1)
    diff = np.abs(got - ref).max(axis=1)
    zero = scale == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float(np.max(diff[~zero] / scale[~zero]))


def state_rel_err(got, ref, lead=2):
    """max over the leading `lead` axes (e.g. batch, head) of max|got - ref| /
    max|ref| over the remaining axes (a whole state at once); an all-zero
    reference must be matched exactly."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    n = int(np.prod(ref.shape[:lead]))
    return row_rel_err(got.reshape(n, -1), ref.reshape(n, -1))


@functools.lru_cache(maxsize=8)
def workload_inputs(name):
    w = gen.WORKLOADS[name]
    if w.kind == "recall":
        q, k, v, g = gen.recall_stream(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype, return_gen=True)
        return w, q, k, v, g
    q, k, v = gen.gaussian_qkv(w.B, w.H, w.T, w.dk, w.dv, w.seed, w.dtype)
    return w, q, k, v, None


def sample_rows(T, C, n_random=24, seed=0):
    """Rows at chunk boundaries, the ends, and random positions."""
    r = np.random.Generator(np.random.PCG64(seed))
    rows = {0, 1, T - 1, T - 2}
    for c in (1, 2, T // C // 2, T // C - 1):
        for off in (-1, 0, 1):
            t = c * C + off
            if 0 <= t < T:
                rows.add(t)
    rows.update(int(x) for x in r.integers(0, T, n_random))
    return np.array(sorted(x for x in rows if 0 <= x < T))
