"""Seeded input generators: determinism, rounding and workload structure (CPU)."""
import numpy as np

from kernelized_linear_attention_phi_amd import inputs as gen


def test_round_to_bf16_is_rne_and_idempotent():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 1e-3, 3.0e38])
    r = gen.round_to(x, "bf16")
    u = r.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    assert r[0] == 1.0 and r[1] == 1.0            # tie rounds to even
    assert r[2] == 1.0 + 2**-7                      # above half rounds up
    assert np.array_equal(gen.round_to(r, "bf16"), r)


def test_gaussian_deterministic_and_unit_rows():
    a = gen.gaussian_qkv(1, 2, 64, 16, 8, seed=7)
    b = gen.gaussian_qkv(1, 2, 64, 16, 8, seed=7)
    c = gen.gaussian_qkv(1, 2, 64, 16, 8, seed=8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    n = np.linalg.norm(a[0].astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 2e-2)


def test_recall_stream_structure():
    q, k, v, g = gen.recall_stream(2, 2, 512, 16, 8, seed=3, return_gen=True)
    assert np.all(v.sum(-1) == 1.0) and set(np.unique(v)) <= {0.0, 1.0}
    # every query repeats an earlier (or the first) key
    for b in range(2):
        for h in range(2):
            kk = k[b, h]
            for t in range(1, 512, 37):
                assert np.any(np.all(kk[:t] == q[b, h, t], axis=-1))
            assert np.array_equal(q[b, h, 0], kk[0])
    # repeated keys with changed values exist (overwrites)
    kk, vv = k[0, 0], v[0, 0].argmax(-1)
    seen = {}
    changed = 0
    for t in range(512):
        key = kk[t].tobytes()
        if key in seen and seen[key] != vv[t]:
            changed += 1
        seen[key] = vv[t]
    assert changed > 50
    dq, dk, dv, src = gen.decode_continuation(g, 2, 4, 16, seed=11)
    assert dq.shape == (16, 4, 2, 16) and dv.shape == (16, 4, 2, 8)
    assert list(src) == [0, 1, 2, 3, 0, 1, 2, 3]
