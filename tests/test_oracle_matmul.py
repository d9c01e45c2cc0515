"""Pins for the oracle's decoded product (EntroPack abstract: the weights are decoded during
inference, for compute-heavy workloads such as Transformer prefill and diffusion denoising).

oracle.decompress_matmul(blob, x) is the plain product Y = X W^T of the blob's decoded tensor W
with an activation block X, in fp64.  It is pinned here to things other than itself:
- unit rows of X pick single columns of W: Y must hold those decoded columns exactly;
- exact rational arithmetic (fractions.Fraction over the decoded container values) on small
  blobs: Y must lie within fp64 summation error of the exact sums, and B (the sum of absolute
  products) within the same bound of its exact value;
- a zero block gives a zero product.
"""

from fractions import Fraction

import numpy as np
import pytest

import ep_synth as S


def _blob(orc, R, C, dt, target=4.0, F=4096, seed=7):
    w = S.iid_normal(R, C, seed, dtype=dt)
    st, blob, _ = orc.compress(w, dt, target, F)
    assert st == 0
    return blob


@pytest.mark.parametrize("dt", [S.BF16, S.FP16])
def test_unit_rows_pick_decoded_columns(orc, dt):
    R, C = 40, 96
    blob = _blob(orc, R, C, dt)
    st, wb, _, _ = orc.decompress(blob)
    assert st == 0
    W = S.container_to_float(wb, dt).astype(np.float64)
    ks = [0, 1, 7, 8, 50, 95]
    X = np.zeros((len(ks), C), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    st, Y, B = orc.decompress_matmul(blob, S.cast_container(X, dt))
    assert st == 0 and Y.shape == (len(ks), R)
    for i, k in enumerate(ks):
        assert np.array_equal(Y[i], W[:, k])
        assert np.array_equal(B[i], np.abs(W[:, k]))


@pytest.mark.parametrize("dt", [S.BF16, S.FP16])
def test_product_matches_exact_rational_sums(orc, dt):
    R, C, m = 24, 64, 3
    blob = _blob(orc, R, C, dt, seed=11)
    st, wb, _, _ = orc.decompress(blob)
    assert st == 0
    W = S.container_to_float(wb, dt)
    xb = S.iid_normal(m, C, 12, sigma=1.0, dtype=dt)
    X = S.container_to_float(xb, dt)
    st, Y, B = orc.decompress_matmul(blob, xb)
    assert st == 0
    u = 2.0 ** -53
    for i in range(m):
        for n in range(R):
            exact = sum(Fraction(float(X[i, k])) * Fraction(float(W[n, k])) for k in range(C))
            babs = sum(abs(Fraction(float(X[i, k])) * Fraction(float(W[n, k])))
                       for k in range(C))
            bound = C * u * float(babs)
            assert abs(Fraction(Y[i, n]) - exact) <= Fraction(bound) + Fraction(1, 2 ** 1074)
            assert abs(Fraction(B[i, n]) - babs) <= Fraction(bound) + Fraction(1, 2 ** 1074)


def test_zero_block(orc):
    blob = _blob(orc, 16, 64, S.BF16)
    st, Y, B = orc.decompress_matmul(blob, np.zeros((5, 64), np.uint16))
    assert st == 0
    assert not Y.any() and not B.any()
