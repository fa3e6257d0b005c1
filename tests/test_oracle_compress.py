"""Pins for the oracle's Compressor (2:1 softmax-gated pooling, NVFP4 article
section 3.2): a closed form, degenerate gates and identical tokens."""
import numpy as np

from oracle import brute
from oracle import csa2_ref as ref


def _bits(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_matches_sigmoid_closed_form():
    rng = np.random.default_rng(11)
    raw = _bits(rng.standard_normal((2, 64, 512)))
    gate = _bits(rng.standard_normal((2, 64, 512)) * 3)
    bits, y = ref.compress(raw, gate)
    exp = brute.compress(raw, gate)
    assert bits.shape == (2, 32, 512)
    np.testing.assert_allclose(y, exp, rtol=1e-12, atol=1e-14)
    # stored bits are the round-to-nearest-even bf16 of the exact value
    for v, b in zip(y.reshape(-1)[:3000], bits.reshape(-1)[:3000]):
        assert ref.round_bf16(v) == int(b)


def test_equal_gates_give_the_mean_exactly():
    rng = np.random.default_rng(12)
    # dyadic inputs: the mean is exact in double and in bf16
    raw = _bits(rng.integers(-64, 64, (1, 16, 512)) / 8.0)
    gate = _bits(np.repeat(rng.standard_normal((1, 8, 1, 512)), 2, axis=1).reshape(1, 16, 512))
    _, y = ref.compress(raw, gate)
    x = brute.dec_bf16(raw)
    assert np.array_equal(y, (x[:, 0::2] + x[:, 1::2]) / 2)


def test_identical_tokens_pass_through():
    rng = np.random.default_rng(13)
    row = rng.standard_normal((1, 1, 512))
    raw = _bits(np.repeat(row, 2, axis=1))
    gate = _bits(rng.standard_normal((1, 2, 512)) * 5)
    bits, _ = ref.compress(raw, gate)
    assert np.array_equal(bits[0, 0], raw[0, 0])


def test_dominant_gate_selects_its_token():
    rng = np.random.default_rng(14)
    raw = _bits(rng.standard_normal((1, 2, 512)))
    gate = np.zeros((1, 2, 512), np.float32)
    gate[0, 0, :256] = 60.0   # token 0 wins on the first half of the channels
    gate[0, 1, 256:] = 60.0   # token 1 wins on the second half
    bits, _ = ref.compress(raw, _bits(gate))
    assert np.array_equal(bits[0, 0, :256], raw[0, 0, :256])
    assert np.array_equal(bits[0, 0, 256:], raw[0, 1, 256:])


def test_pairs_are_consecutive_tokens():
    # latent g pools raw tokens 2g and 2g+1 only: perturbing token 5 moves
    # latent 2 and nothing else
    rng = np.random.default_rng(15)
    raw = _bits(rng.standard_normal((1, 12, 512)))
    gate = _bits(rng.standard_normal((1, 12, 512)))
    a, _ = ref.compress(raw, gate)
    raw2 = raw.copy()
    raw2[0, 5] = _bits(rng.standard_normal(512) + 10)
    b, _ = ref.compress(raw2, gate)
    changed = [g for g in range(6) if not np.array_equal(a[0, g], b[0, g])]
    assert changed == [2]
