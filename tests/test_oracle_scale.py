"""Pins for oracle.scale: hand cases, specials, and the defining property that
the scaled amax lands on e4m3's largest value (448) without saturating
anything finite."""

import numpy as np
import torch

from oracle import e4m3
from oracle import scale as sc


def _bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_hand_cases():
    assert sc.absmax(_bits([1.0, -3.5, 2.0])) == np.float32(3.5)
    assert sc.scale_from_amax(np.float32(3.5)) == np.float32(3.5) / np.float32(448.0)
    assert sc.absmax(_bits([-0.0, 0.0])) == 0.0 and sc.scale_from_amax(0.0) == 1.0
    assert sc.absmax(np.array([], np.uint16)) == 0.0


def test_nan_and_inf_are_ignored():
    x = _bits([1.0, float("nan"), float("inf"), -float("inf"), -2.5])
    assert sc.absmax(x) == np.float32(2.5)
    assert sc.absmax(_bits([float("nan"), float("inf")])) == 0.0


def test_exact_over_all_finite_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        x = e4m3.bf16_bits_to_f32(bits).astype(np.float64)
    fin = np.isfinite(x)
    assert sc.absmax(bits) == np.float32(np.abs(x[fin]).max())        # = the largest finite bf16
    assert sc.absmax(bits) == np.float32(3.3895313892515355e38)


def test_amax_maps_to_448_and_nothing_finite_saturates_past_it():
    rng = np.random.default_rng(1)
    for trial in range(20):
        vals = rng.standard_t(3, 4096).astype(np.float32) * np.float32(10.0 ** rng.uniform(-3, 3))
        bits = _bits(vals)
        a = sc.absmax(bits)
        s = sc.scale_from_amax(a)
        codes = e4m3.quantize(bits, s)
        dec = np.abs(e4m3.decode(codes))
        assert dec.max() == 448.0                                     # the amax element encodes to +-448
        assert np.all(dec <= 448.0)
        amax_pos = np.argmax(np.abs(e4m3.bf16_bits_to_f32(bits)))
        assert abs(e4m3.decode(codes[amax_pos:amax_pos + 1])[0]) == 448.0
