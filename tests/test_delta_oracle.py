"""CPU pins of the DeltaKATA oracle, and planted mistakes in copies of it that
the pins must catch (see tests/delta_checks.py)."""
import inspect
import types

import pytest

import oracle
import oracle.delta_oracle as real
from tests import delta_checks as chk

SRC = inspect.getsource(real)


def _ns(mod):
    return types.SimpleNamespace(brute_force=oracle.brute_force, phi=oracle.phi,
                                 state_from_tokens=oracle.state_from_tokens,
                                 **{n: getattr(mod, n) for n in real.__all__})


MUTATIONS = {
    "erase_sign": ("        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]",
                   "        A = A + beta[:, :, t, None, None] * kt[..., None] * (u + erase)[:, :, None, :]"),
    "no_erase": ("        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]",
                 "        A = A + beta[:, :, t, None, None] * kt[..., None] * u[:, :, None, :]"),
    "beta_on_erase_only": ("        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]",
                           "        A = A + kt[..., None] * (u - beta[:, :, t, None] * erase)[:, :, None, :]"),
    "z_plain_sum": ("        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]",
                    "        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]\n"
                    "        A[..., dv] += kt * (1 - beta[:, :, t, None]) * 0 + kt * erase[..., dv, None] * beta[:, :, t, None]"),
    "readout_before_update": ("        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]\n"
                              "        r = np.einsum(\"bhp,bhpc->bhc\", fq[:, :, t], A)\n",
                              "        r = np.einsum(\"bhp,bhpc->bhc\", fq[:, :, t], A)\n"
                              "        A = A + beta[:, :, t, None, None] * kt[..., None] * (u - erase)[:, :, None, :]\n"),
    "kappa_unnormalised": ("    np.divide(phi(k), n2, out=out, where=n2 != 0.0)",
                           "    np.divide(phi(k), np.ones_like(n2), out=out, where=n2 != 0.0)"),
    "kappa_norm_not_squared": ("    n2 = (k * k).sum(-1, keepdims=True)", "    n2 = np.sqrt((k * k).sum(-1, keepdims=True))"),
    "chunk_mask_strict": ("        W = np.tril(Q @ np.swapaxes(K, -1, -2))                            # j <= t",
                          "        W = np.tril(Q @ np.swapaxes(K, -1, -2), -1)                        # j <= t"),
    "chunk_lower_inclusive": ("        L = np.tril(K @ np.swapaxes(K, -1, -2), -1)", "        L = np.tril(K @ np.swapaxes(K, -1, -2))"),
    "chunk_beta_missing": ("        rhs = b[..., :, None] * (U - K @ A)", "        rhs = U - K @ A"),
    "chunk_state_not_updated": ("        A = A + np.swapaxes(K, -1, -2) @ P", "        A = A + 0.0 * P.sum()"),
    "chunk_prefix_ignored": ("        r = Q @ A + W @ P", "        r = W @ P"),
}


@pytest.mark.parametrize("check", chk.ALL, ids=[c.__name__ for c in chk.ALL])
def test_delta_pin(check):
    check(_ns(real))


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle.delta_mutant")
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), "delta_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_delta_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert chk.failures(_ns(_mutant(old, new))), f"planted mistake {name} passed every pin"
