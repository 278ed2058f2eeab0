"""Seeded input generator: determinism, dtype rounding and the recipe's shapes."""
import numpy as np

from gated_deltanet_chunked_03_amd.synth import make_inputs, round_bf16, CONFIGS


def test_round_bf16_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1e-30, 3.0e38], np.float64)
    r = round_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2**-6 and r[3] == -2.5
    bits = r.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_deterministic_and_normalised():
    a = make_inputs(1, 300, 2, 4, d_k=32, d_v=32, seed=9, gate="mixed")
    b = make_inputs(1, 300, 2, 4, d_k=32, d_v=32, seed=9, gate="mixed")
    for x, y in zip(a.flat(), b.flat()):
        assert np.array_equal(x, y)
    n = np.linalg.norm(a.k.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-2
    assert np.all(round_bf16(a.v) == a.v)
    assert np.all(a.g <= 0) and np.all((a.beta > 0) & (a.beta < 1))
    assert sorted(set(a.head_class)) == ["fast", "slow"]
    assert a.head_class.count("fast") == 3


def test_config_table():
    assert CONFIGS["tp8"]["h_qk"] == 2 and CONFIGS["tp8"]["h_v"] == 8
    assert CONFIGS["long"]["T"] == 262144
    t = make_inputs(**{**CONFIGS["tiny"], "T": 128})
    assert t.io_dtype == "f32" and t.head_class == ["plain"]
