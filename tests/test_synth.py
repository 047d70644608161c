"""The seeded generators: determinism and the structure each workload asks for."""
import numpy as np

import synth


def test_bf16_rounding_once():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 1e-40, 3e38])
    bits = synth.f64_to_bf16_bits(v)
    back = synth.bf16_bits_to_f64(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6
    assert back[3] == -2.5 and back[4] == 0.0
    assert abs(back[5] - 1e-40) <= 2.0 ** -134


def test_deterministic():
    a = synth.gen_c3(8)["a"]
    b = synth.gen_c3(8)["a"]
    assert np.array_equal(a, b)
    assert not np.array_equal(synth.gen_c3(8)["a"][:1], synth.gen_c3(1)["a"])


def test_c1_structure():
    d = synth.gen_c1()
    a = synth.bf16_bits_to_f64(d["a"])
    assert d["a"].shape == (32, 512) and d["w"].shape == (512, 512)
    assert np.all(a.reshape(-1, 128)[d["zero_block"]] == 0)
    assert np.count_nonzero(np.abs(a) > 10) > 100       # the x50 entries


def test_c5_structure():
    d = synth.gen_c5(M=1024)                              # same recipe, fewer rows
    a = synth.bf16_bits_to_f64(d["a"]).reshape(-1, 128)
    assert np.all(a[d["zero_blocks"]] == 0)
    assert np.all(np.max(np.abs(a[d["big_blocks"]]), axis=1) >= 1e4)
    assert d["w_scale"].dtype == np.float32
    assert d["w_scale"].min() >= 1e-4 * 0.999 and d["w_scale"].max() <= 1e-1 * 1.001


def test_quotient_grid_covers_all_significand_pairs():
    g = synth.quotient_grid(amax_exponents=(0,))
    amax_sig = g[:, 0] & 0x7F
    assert set(amax_sig.tolist()) == set(range(128))
    x = g[:, 1:] & 0x7FFF
    assert np.all(x <= (g[:, :1] & 0x7FFF))
