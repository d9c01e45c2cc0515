"""Pins for the oracle's row normalisation (design page "EntroPack lattice compression",
*Lattice quantization and integer fields*: every row is first divided by its root mean square).

The oracle's reading: sumsq_r = sum of the widened squares in fp64, accumulated left to right
over the row's real elements (cols of them, also when cols % 8 != 0); rms_r = sqrt(sumsq_r / cols);
gain g_r = fp32(1 / (rms_r * s)), and 0 for a row of zeros.

Nothing here calls the oracle's own widening or retypes its formula.  The checks are:
  * hand-worked rows whose RMS is known in closed form (all 2.0 -> 2; +-1 alternating -> 1;
    a 13-element row [3, 4, 0, ...] -> sqrt(25 / 13), which a denominator of 16 would miss);
  * the summation order: 2^60 followed by 1024 ones stays at 2^60 when added left to right,
    while the same terms in the other order reach 2^60 + 1024 exactly;
  * numpy's sequential cumulative sum of the squares (widened by torch / numpy casts), bit for
    bit, in every container at ragged widths, and the classical bound of a recursive sum against
    math.fsum (relative error at most (n - 1) 2^-53);
  * the gain against 1 / (sqrt(sumsq / C) s) evaluated to 60 significant digits and rounded once
    to fp32: the oracle's fp64 steps must give that correctly rounded value except within 2^-45
    of an fp32 rounding boundary (none occur in these draws).  A gain rounded to fp32 twice, an
    fp32 square root, or a mean absolute value in place of the RMS all fail this.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import ep_synth as S

DTYPES = [S.BF16, S.FP16, S.FP8, S.INT8, S.FP32]


def _row(vals, dt):
    return S.cast_container(np.asarray(vals, np.float32).reshape(1, -1), dt)


def test_hand_worked_rows(orc):
    # all 2.0: sumsq = 4 C, rms = 2, gain at s = 0.5 is exactly 1
    w = _row([2.0] * 64, S.BF16)
    ss = orc.row_sumsq(w, S.BF16)
    assert ss[0] == 256.0
    assert orc.gains(ss, 64, 0.5)[0] == np.float32(1.0)
    # +-1 alternating: rms 1, gain at s = 0.25 is 4
    w = _row([1.0, -1.0] * 8, S.FP16)
    ss = orc.row_sumsq(w, S.FP16)
    assert ss[0] == 16.0
    assert orc.gains(ss, 16, 0.25)[0] == np.float32(4.0)
    # a ragged row of 13 real elements: rms = sqrt(25 / 13) (not over 16 padded elements)
    w = _row([3.0, 4.0] + [0.0] * 11, S.INT8)
    ss = orc.row_sumsq(w, S.INT8)
    assert ss[0] == 25.0
    g = orc.gains(ss, 13, 1.0)[0]
    assert g == np.float32(math.sqrt(13.0) / 5.0)
    assert g != np.float32(math.sqrt(16.0) / 5.0)
    # a zero row: sum 0, gain 0 (not inf or NaN)
    w = _row([0.0] * 24, S.BF16)
    ss = orc.row_sumsq(w, S.BF16)
    assert ss[0] == 0.0
    assert orc.gains(ss, 24, 0.1)[0] == np.float32(0.0)


def test_left_to_right_order(orc):
    big = float(2.0 ** 30)
    w = _row([big] + [1.0] * 1024, S.FP32)
    assert orc.row_sumsq(w, S.FP32)[0] == 2.0 ** 60            # every +1 rounds away
    w = _row([1.0] * 1024 + [big], S.FP32)
    assert orc.row_sumsq(w, S.FP32)[0] == 2.0 ** 60 + 1024.0   # the ones add up first


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("cols", [8, 13, 1001, 4096])
def test_sumsq_matches_sequential_numpy_sum(orc, dt, cols):
    rng = np.random.Generator(np.random.PCG64(7100 + 10 * dt + cols))
    rows = 12
    scale = 40.0 if dt == S.INT8 else 0.02
    vals = rng.standard_normal((rows, cols)) * scale * np.exp(rng.normal(0, 1.0, (rows, 1)))
    w = S.cast_container(vals.astype(np.float32), dt)
    got = orc.row_sumsq(w, dt)
    v = S.container_to_float(w, dt).astype(np.float64)
    seq = np.cumsum(v * v, axis=1)[:, -1]                       # left to right, squares exact
    assert np.array_equal(got, seq)
    for r in range(rows):
        exact = math.fsum((v[r] * v[r]).tolist())
        assert abs(got[r] - exact) <= (cols - 1) * 2.0 ** -53 * exact


def _exact_gain(sumsq: float, cols: int, s: float) -> Decimal:
    getcontext().prec = 60
    rms = (Decimal(sumsq) / Decimal(cols)).sqrt()
    return Decimal(1) / (rms * Decimal(s))


def _fp32_neighbours(x: Decimal):
    """The two fp32 values around x > 0 and the midpoint between them, as Decimals."""
    f = np.float32(float(x))
    lo = f if Decimal(float(f)) <= x else np.nextafter(f, np.float32(0))
    hi = np.nextafter(lo, np.float32(np.inf))
    return lo, hi, (Decimal(float(lo)) + Decimal(float(hi))) / 2


def test_gain_is_the_correctly_rounded_fp32(orc):
    rng = np.random.Generator(np.random.PCG64(7203))
    checked = 0
    for i in range(3000):
        cols = int(rng.integers(1, 30000))
        sumsq = float(np.exp(rng.uniform(-40, 25)))
        s = float(2.0 ** rng.uniform(-20, 12))
        g = orc.gains(np.array([sumsq]), cols, s)[0]
        ex = _exact_gain(sumsq, cols, s)
        lo, hi, mid = _fp32_neighbours(ex)
        if abs(ex - mid) <= ex * Decimal(2) ** -45:
            continue                                           # too close to call: skipped
        want = lo if ex < mid else hi
        assert g == want, (cols, sumsq, s, g, want)
        checked += 1
    assert checked >= 2990


def test_gain_of_real_rows_in_every_container(orc):
    """Rows drawn like the workloads, with the RMS over the real elements of ragged widths."""
    for dt in DTYPES:
        for cols in (13, 200):
            w = S.workload_weights(2, rows=6, cols=cols) if dt == S.BF16 else S.cast_container(
                (np.random.Generator(np.random.PCG64(dt)).laplace(0, 0.01, (6, cols)) *
                 (5000.0 if dt == S.INT8 else 1.0)).astype(np.float32), dt)
            ss = orc.row_sumsq(w, dt)
            v = S.container_to_float(w, dt).astype(np.float64)
            for r in range(w.shape[0]):
                s = 0.37
                g = orc.gains(ss[r:r + 1], cols, s)[0]
                ex = _exact_gain(float(ss[r]), cols, s)
                lo, hi, mid = _fp32_neighbours(ex)
                want = lo if ex < mid else hi
                assert g == want
                # the gain normalises the row: its RMS times s times g is 1 to fp32 precision
                rms = math.sqrt(math.fsum((v[r] * v[r]).tolist()) / cols)
                assert abs(float(g) * rms * s - 1.0) < 2.0 ** -22
