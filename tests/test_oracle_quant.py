"""Pins of the oracle's residual quantizer (CPU only).

The quantizer reading (FlashLoop abstract, third observation: low-bit KV
residuals) is pinned by hand-worked groups, the round-trip error bound, exact
dequantization, scale equivariance and the int4 packing layout.
"""
import json
import os

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked_examples.json")


def _group(vals):
    r = np.zeros(32, np.float32)
    r[: len(vals)] = np.asarray(vals, np.float32)
    return r


def test_worked_examples():
    data = json.load(open(GOLDEN))
    for case in data["cases"]:
        r = _group(case["r"])
        codes, s16 = quant.quantize(r, case["bits"])
        assert s16.shape == (1,)
        assert float(s16[0]) == pytest.approx(case["scale_f16"], rel=0, abs=0), case["comment"]
        exp = np.zeros(32, np.int8)
        exp[: len(case["codes"])] = case["codes"]
        np.testing.assert_array_equal(codes, exp, err_msg=case["comment"])


def test_int4_packing_layout():
    data = json.load(open(GOLDEN))["int4_packing"]
    codes = np.asarray(data["codes"], np.int8)
    packed = quant.pack_int4(codes)
    np.testing.assert_array_equal(packed, np.asarray(data["bytes"], np.uint8))
    np.testing.assert_array_equal(quant.unpack_int4(packed), codes)


@pytest.mark.parametrize("bits", [4, 8])
def test_round_trip_bound_and_range(bits):
    rng = np.random.default_rng(5)
    qmax = 2 ** (bits - 1) - 1
    # rows spanning many magnitudes; 64 elements = 2 groups per row
    mags = np.float32(10.0) ** rng.uniform(-4, 3, size=(4000, 1)).astype(np.float32)
    r = (rng.standard_normal((4000, 64)).astype(np.float32) * mags).astype(np.float32)
    codes, s16 = quant.quantize(r, bits)
    assert codes.min() >= -qmax and codes.max() <= qmax
    deq = quant.dequantize(codes, s16)
    s = s16.astype(np.float32)
    normal = s >= np.float32(2.0 ** -14)
    err = np.abs(r - deq).reshape(4000, 2, 32)
    bound = (s / 2)[..., None]
    assert np.all(err[normal] <= bound[normal])
    # the largest-magnitude element of every group maps to +-qmax
    g = r.reshape(4000, 2, 32)
    am = np.argmax(np.abs(g), axis=-1)
    c = codes.reshape(4000, 2, 32)
    top = np.take_along_axis(c, am[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top[normal]) == qmax)


def test_dequant_is_exact_product():
    rng = np.random.default_rng(7)
    r = rng.standard_normal((100, 128)).astype(np.float32)
    codes, s16 = quant.quantize(r, 8)
    deq = quant.dequantize(codes, s16)
    exact = codes.astype(np.float64).reshape(100, 4, 32) * s16.astype(np.float64)[..., None]
    np.testing.assert_array_equal(deq.astype(np.float64), exact.reshape(100, 128))


@pytest.mark.parametrize("bits", [4, 8])
def test_power_of_two_equivariance(bits):
    rng = np.random.default_rng(11)
    r = rng.standard_normal((500, 32)).astype(np.float32)
    c0, s0 = quant.quantize(r, bits)
    for m in (-3, 2, 5):
        c1, s1 = quant.quantize(r * np.float32(2.0 ** m), bits)
        np.testing.assert_array_equal(c0, c1)
        np.testing.assert_array_equal(s1.astype(np.float32), s0.astype(np.float32) * np.float32(2.0 ** m))


def test_zero_group_and_bad_sizes():
    codes, s16 = quant.quantize(np.zeros((3, 64), np.float32), 4)
    assert not codes.any() and not s16.astype(np.float32).any()
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((2, 48), np.float32), 4)
    with pytest.raises(ValueError):
        quant.qmax_of(6)
