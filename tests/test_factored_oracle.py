"""CPU pins of the KATA-Mg / KATA-Sigma-g oracle, and planted mistakes in copies
of it that the pins must catch (see tests/factored_checks.py)."""
import inspect
import types

import pytest

import oracle
import oracle.factored_oracle as real
from tests import factored_checks as chk

SRC = inspect.getsource(real)


def _ns(mod):
    return types.SimpleNamespace(brute_force=oracle.brute_force, phi=oracle.phi,
                                 state_from_tokens=oracle.state_from_tokens,
                                 **{n: getattr(mod, n) for n in real.__all__})


MUTATIONS = {
    # factors interleaved (x[a::g]) instead of contiguous
    "factors_interleaved": (
        "    return x.reshape(x.shape[:-1] + (g, x.shape[-1] // g))",
        "    return np.swapaxes(x.reshape(x.shape[:-1] + (x.shape[-1] // g, g)), -1, -2)"),
    # multi summed like Sigma-g
    "multi_features_summed": (
        "    if kind == \"multi\":\n        return lifts.reshape(lifts.shape[:-2] + (-1,))\n",
        "    if kind == \"multi\":\n        return lifts.sum(axis=-2)\n"),
    # Sigma-g without the cross-factor products
    "summed_no_cross_terms": (
        "    return (dots ** 2).sum(axis=(-2, -1))",
        "    return (np.diagonal(dots, axis1=-2, axis2=-1) ** 2).sum(-1)"),
    # squares of sums instead of sums of squares
    "multi_square_of_sum": (
        "        return (np.diagonal(dots, axis1=-2, axis2=-1) ** 2).sum(-1)",
        "        return np.diagonal(dots, axis1=-2, axis2=-1).sum(-1) ** 2"),
    "summed_square_of_sum": (
        "    return (dots ** 2).sum(axis=(-2, -1))",
        "    return dots.sum(axis=(-2, -1)) ** 2"),
    "weights_not_squared": (
        "    return (dots ** 2).sum(axis=(-2, -1))",
        "    return np.abs(dots).sum(axis=(-2, -1))"),
    "prior_ignored": (
        "    pn, pd = _prior(q_rows, g, kind, S0, z0)\n",
        "    pn, pd = 0.0, 0.0\n"),
    "recurrent_reads_before_update": (
        "        S += fk[:, :, t, :, None] * v[:, :, t, None, :]\n        z += fk[:, :, t]\n"
        "        o[:, :, t] = _safe_ratio(np.einsum(\"bhp,bhpn->bhn\", fq[:, :, t], S),\n"
        "                                 np.einsum(\"bhp,bhp->bh\", fq[:, :, t], z))\n",
        "        o[:, :, t] = _safe_ratio(np.einsum(\"bhp,bhpn->bhn\", fq[:, :, t], S),\n"
        "                                 np.einsum(\"bhp,bhp->bh\", fq[:, :, t], z))\n"
        "        S += fk[:, :, t, :, None] * v[:, :, t, None, :]\n        z += fk[:, :, t]\n"),
    "chunk_mask_strict": (
        "        A = factored_weights(Qc, Kc, g, kind) * np.tril(np.ones((n, n)))",
        "        A = factored_weights(Qc, Kc, g, kind) * np.tril(np.ones((n, n)), -1)"),
    "chunk_state_not_carried": (
        "        S, z = S + Sc, z + zc\n    return o, S, z",
        "        S, z = Sc, zc\n    return o, S, z"),
    "decode_reads_old_state": (
        "    return (_safe_ratio(np.einsum(\"np,npv->nv\", fq, S2), np.einsum(\"np,np->n\", fq, z2)), S2, z2)",
        "    return (_safe_ratio(np.einsum(\"np,npv->nv\", fq, np.asarray(S, np.float64)),\n"
        "                        np.einsum(\"np,np->n\", fq, np.asarray(z, np.float64))), S2, z2)"),
    "dim_multi_wrong": (
        "    return g * phi_dim(p) if kind == \"multi\" else phi_dim(p)",
        "    return phi_dim(p) if kind == \"multi\" else g * phi_dim(p)"),
}


@pytest.mark.parametrize("check", chk.ALL, ids=[c.__name__ for c in chk.ALL])
def test_factored_pin(check):
    check(_ns(real))


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle.factored_mutant")
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), "factored_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_factored_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert chk.failures(_ns(_mutant(old, new))), f"planted mistake {name} passed every pin"
