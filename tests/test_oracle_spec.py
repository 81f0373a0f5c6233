"""Pins for the oracle's softmax-weight arithmetic and row statistics.

The oracle's confidences are the draft softmax probabilities (EAGLE-2
explainer, "Draft model calibration").  The arithmetic that makes them exactly
reproducible is checked here against: exact rational values of its constants,
the true exponential (error bound), an independent vectorised emulation of
the same IEEE steps, exact integer sums, and a library sort for the top-C order.
"""
import math
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import spec_emul

pytestmark = []


def _f32_bits(v):
    return struct.unpack(">I", struct.pack(">f", float(v)))[0]


def test_constants_are_rn32_of_exact_series():
    # 2^f = sum_j (f ln2)^j / j!; coefficients rounded once to float32
    getcontext().prec = 80
    ln2 = Fraction(Decimal(2).ln())
    expected = [0x3F800000, 0x3F317218, 0x3E75FDF0, 0x3D635847, 0x3C1D955B, 0x3AAEC3FF, 0x39218489]
    got = [_f32_bits(spec_emul.rn32_fraction(ln2 ** j / math.factorial(j))) for j in range(7)]
    assert got == expected
    assert _f32_bits(spec_emul.rn32_fraction(1 / ln2)) == 0x3FB8AA3B


def test_exp_spec_matches_true_exp_within_bound(orc):
    xs = np.concatenate([np.linspace(-32, 0, 20001, dtype=np.float32),
                         -np.logspace(-8, 1.5, 2001).astype(np.float32)])
    got = orc.exp_spec(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    rel = np.abs(got - ref) / ref
    assert rel.max() < 2.5e-6
    assert orc.exp_spec(np.float32(0.0)) == 1.0
    assert orc.exp_spec(np.float32(-0.0)) == 1.0
    assert (got <= 1.0).all()


def test_exp_spec_bit_exact_vs_independent_emulation(orc):
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.uniform(-40, 0, 4000).astype(np.float32),
                         np.float32([-0.5, -1.5, -0.0, 0.0, -32.0, -31.999998, -1e-30, -24.26])])
    got = orc.exp_spec(xs)
    ref = spec_emul.exp_spec(xs)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_weights_bit_exact_vs_emulation_and_integer_properties(orc):
    rng = np.random.default_rng(2)
    l = (rng.standard_normal(3000) * 3).astype(np.float32)
    M = np.float32(l.max())
    emu = spec_emul.weights(l, M)
    got = np.array([orc.weight(v, M) for v in l])
    assert np.array_equal(got, emu)
    assert np.all(got == np.floor(got)) and got.min() >= 0 and got.max() == 2.0 ** 35
    # temperature path: x = (l - M) / T in float32
    emuT = spec_emul.weights(l, M, T=0.7)
    gotT = np.array([orc.weight(v, M, 0.7) for v in l])
    assert np.array_equal(gotT, emuT)


def test_weight_tail_is_zero_and_nan_propagates(orc):
    assert orc.weight(-25.0, 0.0) == 0.0
    assert orc.weight(-1e30, 0.0) == 0.0
    assert orc.weight(float("-inf"), 0.0) == 0.0
    assert math.isnan(orc.weight(float("nan"), 0.0))
    # largest x with a nonzero weight: exp(x) * 2^35 >= 1  <=>  x >= -35 ln 2 = -24.26
    assert orc.weight(-24.0, 0.0) > 0


@pytest.mark.parametrize("V,C,dtype", [(1000, 10, "f32"), (32000, 10, "bf16"), (37, 16, "bf16")])
def test_row_stats_exact_sum_and_library_order(orc, V, C, dtype):
    rng = np.random.default_rng(V)
    rows = (rng.standard_normal((6, V)) * 3).astype(np.float32)
    if dtype == "bf16":
        import torch
        rows = torch.from_numpy(rows).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    M, W, tid, tw = orc.row_stats(rows, C)
    for r in range(rows.shape[0]):
        eM, eW, eids, ew = spec_emul.row_stats(rows[r], C)
        assert M[r] == eM
        assert int(W[r]) == eW and float(W[r]) == float(eW)   # exact integer sum
        assert list(tid[r]) == list(eids)
        assert [int(v) for v in tw[r]] == ew


def test_row_stats_ties_and_signed_zero(orc):
    # all-equal row: top-C are ids 0..C-1, W = V * 2^35
    row = np.zeros((1, 50), np.float32)
    M, W, tid, tw = orc.row_stats(row, 5)
    assert list(tid[0]) == [0, 1, 2, 3, 4] and W[0] == 50 * 2.0 ** 35
    # -0 and +0 are equal keys: ties broken by id
    row = np.array([[-1.0, -0.0, 0.0, -0.0, -2.0]], np.float32)
    _, _, tid, _ = orc.row_stats(row, 3)
    assert list(tid[0]) == [1, 2, 3]


def test_row_stats_flags_nonfinite(orc):
    row = np.zeros((1, 10), np.float32)
    row[0, 3] = np.inf
    with pytest.raises(orc.OracleError):
        orc.row_stats(row, 2)
    row[0, 3] = np.nan
    with pytest.raises(orc.OracleError):
        orc.row_stats(row, 2)
