"""CPU pins of the decay-gated oracle, and planted mistakes in copies of it that
the pins must catch (see tests/decay_checks.py)."""
import inspect
import types

import pytest

import oracle
import oracle.decay_oracle as real
from tests import decay_checks as chk

SRC = inspect.getsource(real)


def _ns(mod):
    return types.SimpleNamespace(brute_force=oracle.brute_force, prefix_states=oracle.prefix_states,
                                 fo_brute_force=oracle.fo_brute_force,
                                 fo_state_from_tokens=oracle.fo_state_from_tokens,
                                 **{n: getattr(mod, n) for n in real.__all__})


MUTATIONS = {
    "decay_after_add": ("        S = gam[:, :, None, None] * S + fk[:, :, t, :, None] * v[:, :, t, None, :]\n",
                        "        S = gam[:, :, None, None] * (S + fk[:, :, t, :, None] * v[:, :, t, None, :])\n"),
    "den_not_decayed": ("        z = gam[:, :, None] * z + fk[:, :, t, :]\n", "        z = z + fk[:, :, t, :]\n"),
    "exclusive_cumsum": ("            diff = np.where(mask, G[b, h][:, None] - G[b, h][None, :], -np.inf)",
                         "            diff = np.where(mask, G[b, h][:, None] - G[b, h][None, :] - g[b, h][:, None], -np.inf)"),
    "initial_state_not_decayed": ("                e = np.exp(G[b, h])[:, None]", "                e = np.ones_like(G[b, h])[:, None]"),
    "combine_swapped": ("return a1 * a2, a2[..., None, None] * S1 + S2, a2[..., None] * z1 + z2",
                        "return a1 * a2, a1[..., None, None] * S2 + S1, a1[..., None] * z2 + z1"),
    "inter_not_scaled": ("        num = np.einsum(\"bhtj,bhjn->bhtn\", A, Vc) + e[..., None] * np.einsum(",
                         "        num = np.einsum(\"bhtj,bhjn->bhtn\", A, Vc) + 1.0 * np.einsum("),
    "chunk_weight_inverted": ("    wgt = np.exp(G[..., -1:] - G)", "    wgt = np.exp(G - G[..., -1:])"),
    "chunk_decay_exclusive": ("    return np.exp(G[..., -1]), S, fk.sum(axis=2)",
                              "    return np.exp(G[..., -1] - np.asarray(g, np.float64)[..., 0]), S, fk.sum(axis=2)"),
    "decode_no_decay": ("    gam = np.exp(np.asarray(g, np.float64))\n", "    gam = np.ones_like(np.asarray(g, np.float64))\n"),
    "rows_weight_sign": ("np.exp(G[b, h, t] - G[b, h, :t + 1])", "np.exp(G[b, h, :t + 1] - G[b, h, t])"),
    "intra_mask_strict": ("        tri = np.tril(np.ones((n, n), dtype=bool))", "        tri = np.tril(np.ones((n, n), dtype=bool), -1)"),
    "identity_weight_squared": ('    return s ** 2 if feature == "psd" else s', "    return s ** 2"),
    "identity_lift_scaled": ('    if feature == "identity":\n        return np.asarray(x, np.float64)',
                             '    if feature == "identity":\n        return 2.0 * np.asarray(x, np.float64)'),
}


@pytest.mark.parametrize("check", chk.ALL, ids=[c.__name__ for c in chk.ALL])
def test_decay_pin(check):
    check(_ns(real))


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle.decay_mutant")
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), "decay_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_decay_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert chk.failures(_ns(_mutant(old, new))), f"planted mistake {name} passed every pin"
