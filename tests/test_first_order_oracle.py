"""CPU pins of the first-order oracle, and planted mistakes in copies of it
that the pins must catch (see tests/first_order_checks.py)."""
import inspect
import types

import pytest

import oracle
import oracle.first_order_oracle as real
from tests import first_order_checks as chk

SRC = inspect.getsource(real)


def _ns(mod):
    return types.SimpleNamespace(phi=oracle.phi, brute_force=oracle.brute_force,
                                 **{n: getattr(mod, n) for n in real.__all__})


MUTATIONS = {
    "squared_weights": ("w = q[b, h] @ k[b, h].T ", "w = (q[b, h] @ k[b, h].T) ** 2 "),
    "exclusive_mask": ("w = w * np.tril(np.ones((T, T)))", "w = w * np.tril(np.ones((T, T)), -1)"),
    "prior_den_dropped": ("                den = den + q[b, h] @ np.asarray(z0[b, h], np.float64)\n", ""),
    "read_before_update": ("        S += k[:, :, t, :, None] * v[:, :, t, None, :]\n        z += k[:, :, t, :]\n",
                           ""),
    "z_from_values": ("return S, k.sum(axis=2)", "return S, np.asarray(v, np.float64).sum(axis=2)"),
    "chunk_state_first": ("        num = np.einsum(\"bhtj,bhjn->bhtn\", A, Vc) + np.einsum(\"bhta,bhan->bhtn\", Qc, S)\n",
                          "        S = S + fo_state_from_tokens(Kc, Vc)[0]\n        num = np.einsum(\"bhtj,bhjn->bhtn\", A, Vc) + np.einsum(\"bhta,bhan->bhtn\", Qc, S)\n"),
    "chunk_transposed": ('A = np.einsum("bhta,bhja->bhtj", Qc, Kc)', 'A = np.einsum("bhta,bhja->bhtj", Kc, Qc)'),
    "chunk_den_axis": ("den = A.sum(axis=-1) +", "den = A.sum(axis=-2) +"),
    "zero_rule_broken": ("out = np.zeros(np.broadcast_shapes", "out = np.ones(np.broadcast_shapes"),
    "noncausal_no_S0": ("        S, z = S + St, z + zt\n", "        S, z = St, zt\n"),
}


@pytest.mark.parametrize("check", chk.ALL, ids=[c.__name__ for c in chk.ALL])
def test_first_order_pin(check):
    check(_ns(real))


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("fo_mutant")
    exec(compile(SRC.replace(old, new), "fo_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_first_order_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert chk.failures(_ns(_mutant(old, new))), f"planted mistake {name} passed every pin"
