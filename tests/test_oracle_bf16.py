"""Pins for the oracle's bf16 rounding (CPU only).

* Hand-derived bit patterns, including ties to even.
* A value where rounding through float32 first would give a different
  answer (the oracle rounds float64 directly).
* For float32-representable inputs, torch's float32 -> bfloat16 conversion
  (a library routine, round-to-nearest-even) must agree exactly.
"""
import numpy as np
import torch

from oracle import bf16


def test_hand_bits():
    cases = {
        1.0: 0x3F80, -2.5: 0xC020, 0.0: 0x0000,
        1.0 + 2.0 ** -8: 0x3F80,            # halfway, rounds to even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # halfway, rounds to even (up)
        2.640625: 0x4029, 5.28125: 0x40A9,
    }
    for v, bits in cases.items():
        assert int(bf16.to_bits(np.array([v]))[0]) == bits, (v, hex(bits))


def test_no_double_rounding():
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30        # just above the halfway point
    assert int(bf16.to_bits(np.array([v]))[0]) == 0x3F81
    # via float32 this would land exactly on the halfway point and go to 0x3F80
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)


def test_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # add exact halfway points between neighbouring bf16 values
    base = (rng.integers(0x3000, 0x4F00, 5000).astype(np.uint32) << 16)
    half = (base | 0x8000).view(np.float32)
    v = np.concatenate([v, half, -half, np.float32([1e-39, 3e38])])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.to_bits(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_roundtrip_and_ulp_distance():
    b = np.array([0x3F80, 0x3F81, 0xBF80, 0x0000, 0x8000], dtype=np.uint16)
    assert np.array_equal(bf16.to_bits(bf16.from_bits(b)), np.array([0x3F80, 0x3F81, 0xBF80, 0, 0x8000], np.uint16))
    d = bf16.ulp_distance(np.array([0x3F80, 0x0000, 0x0001], np.uint16),
                          np.array([0x3F81, 0x8000, 0x8001], np.uint16))
    assert d.tolist() == [1, 0, 2]
