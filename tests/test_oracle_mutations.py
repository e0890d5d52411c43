"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins in tests/oracle_checks.py catch every one of them."""
import inspect
import types

import pytest

import oracle.kata_oracle as real
from tests import oracle_checks as chk

SRC = inspect.getsource(real)

MUTATIONS = {
    "no_sqrt2": ("scale = 1.0 if i == j else SQRT2", "scale = 1.0"),
    "phi_wrong_index": ("scale * x[..., i] * x[..., j]", "scale * x[..., i] * x[..., i]"),
    "exclusive_mask": ("<= t_idx[:, None]", "< t_idx[:, None]"),
    "weights_not_squared": ("w = (q_rows @ k.T) ** 2", "w = np.abs(q_rows @ k.T)"),
    "prior_dropped_from_den": ("_safe_ratio(num + pn, den + pd)", "_safe_ratio(num + pn, den)"),
    "strict_intra_mask": ("np.tril(np.ones((n, n)))", "np.tril(np.ones((n, n)), -1)"),
    "transposed_intra": ('"bhtd,bhjd->bhtj", Qc, Kc', '"bhtd,bhjd->bhtj", Kc, Qc'),
    "intra_den_wrong_axis": ("den = A.sum(axis=-1)", "den = A.sum(axis=-2)"),
    "recurrent_stale_value": ("S += fk[:, :, t, :, None] * v[:, :, t, None, :]",
                              "S += fk[:, :, t, :, None] * v[:, :, t - 1, None, :]"),
    "decode_z_from_query": ("z2 = np.asarray(z, np.float64) + fk", "z2 = np.asarray(z, np.float64) + fq"),
    "zero_rule_broken": ("out = np.zeros(np.broadcast_shapes", "out = np.ones(np.broadcast_shapes"),
    "ragged_chunk_drop": ("state_from_tokens(k[:, :, c * C:(c + 1) * C], v[:, :, c * C:(c + 1) * C])",
                          "state_from_tokens(k[:, :, c * C:(c + 1) * C - 1], v[:, :, c * C:(c + 1) * C - 1])"),
    "inclusive_prefix": ("        P[:, :, c] = S\n        Z[:, :, c] = z\n",
                         "        P[:, :, c] = S + state_from_tokens(k[:, :, c * C:(c + 1) * C], v[:, :, c * C:(c + 1) * C])[0]\n        Z[:, :, c] = z\n"),
    "z_abs": ("return S, fk.sum(axis=2)", "return S, np.abs(fk).sum(axis=2)"),
    "noncausal_ignores_S0": ("            S = S + S0\n", "            S = S0\n"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_passes_all():
    assert chk.failures(real) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    caught = chk.failures(_mutant(old, new))
    assert caught, f"planted mistake {name} passed every pin"
