"""Pins for the oracle's E8 quantiser and field map (EntroPack design page, "Lattice
quantization and integer fields").

- hand-worked cases (tests/golden/e8_cases.txt);
- brute force: the fast quantiser's point is as close as the best of 2 x 3^8 enumerated
  candidates (exact long-double distances);
- certificate: no E8 root r (the 240 Voronoi-relevant vectors) moves the point closer;
- second moment: for uniform inputs the mean squared error per coordinate tends to
  G(E8) = 929/12960 (E8 here has unit covolume; Conway & Sloane, SPLAG ch. 21);
- lattice invariants: both cosets give a D8 point z (even coordinate sum);
- field map: exhaustive bijection on D8 inside [-3, 3]^8.
"""

import os

import numpy as np
import pytest

import ep_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e8_cases.txt")
G_E8 = 929.0 / 12960.0


def golden_cases():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        x, c, z, f, note = [p.strip() for p in line.split("|")]
        out.append((np.array(x.split(), np.float32), int(c), np.array(z.split(), np.int32),
                    np.array(f.split(), np.int32), note))
    return out


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c[4])
def test_golden_cases(orc, case):
    x, c, z, f, _ = case
    cc, zz = orc.e8_nearest(x[None, :])
    assert int(cc[0]) == c
    assert np.array_equal(zz[0], z)
    ff = orc.fields_from_point(c, z)
    assert np.array_equal(ff, f)
    assert np.array_equal(orc.point_from_fields(f), z)
    # the brute-force minimum distance equals the chosen point's distance
    _, _, dmin = orc.e8_brute(x)
    p = z.astype(np.float64) + 0.5 * c
    assert abs(float(np.sum((x.astype(np.float64) - p) ** 2)) - dmin) < 1e-12


def _rand_vectors(n, scale, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((n, 8)) * scale).astype(np.float32)


@pytest.mark.parametrize("scale", [0.3, 1.0, 3.0, 40.0])
def test_fast_equals_brute_force(orc, scale):
    x = np.ascontiguousarray(_rand_vectors(1500, scale, seed=int(scale * 10)))
    bad = orc.lib().or_e8_vs_brute(orc._p(x), x.shape[0], 1e-6)
    assert bad == 0


def test_fast_equals_brute_force_on_half_grid(orc):
    # inputs on the quarter-integer grid hit many exact ties between candidates
    g = np.random.Generator(np.random.PCG64(7))
    x = np.ascontiguousarray((g.integers(-8, 9, (2000, 8)) * 0.25).astype(np.float32))
    bad = orc.lib().or_e8_vs_brute(orc._p(x), x.shape[0], 0.0)
    assert bad == 0


def test_root_certificate(orc):
    x = np.ascontiguousarray(_rand_vectors(200_000, 5.0, seed=11))
    bad = orc.lib().or_e8_certificate(orc._p(x), x.shape[0], 1e-6, None)
    assert bad == 0


def test_second_moment_is_G_E8(orc):
    g = np.random.Generator(np.random.PCG64(3))
    x = np.ascontiguousarray(g.uniform(-50, 50, (300_000, 8)).astype(np.float32))
    mse = orc.lib().or_e8_mse(orc._p(x), x.shape[0])
    assert abs(mse - G_E8) / G_E8 < 0.01
    # D8 alone (coset 0 only) would give G(D8) * 2^(1/4) ~ 0.0911, Z^8 1/12 ~ 0.0833


def test_lattice_invariants_and_fields(orc):
    x = _rand_vectors(20_000, 4.0, seed=5)
    c, z = orc.e8_nearest(x)
    assert np.all(z.sum(axis=1) % 2 == 0)          # z in D8 for both cosets
    p = z + 0.5 * c[:, None]
    half = c == 1
    assert np.all(np.abs(p[half] - np.floor(p[half]) - 0.5) == 0)   # all half-integers
    assert np.all(p[~half] == np.floor(p[~half]))                    # all integers
    assert np.all(np.sum(p, axis=1) % 2 == 0)                        # even coordinate sum


def test_field_map_bijection_box(orc):
    assert orc.lib().or_field_bijection_box(3) == 0


def test_field_map_large_values(orc):
    g = np.random.Generator(np.random.PCG64(9))
    for _ in range(2000):
        z = g.integers(-32767, 32768, 8).astype(np.int32)
        if z.sum() % 2:
            z[7] += -1 if z[7] > 0 else 1
        f = orc.fields_from_point(0, z)
        assert f[7] == z[7] // 2
        assert np.array_equal(orc.point_from_fields(f), z)


def test_quantize_rows_are_nearest_points(orc):
    """or_quantize applies x = fp32(w) * g per row and snaps each 8-vector of the row."""
    w = S.lognormal_rows(16, 64, seed=21)
    ss = orc.row_sumsq(w, S.BF16)
    g = orc.gains(ss, 64, 0.25)
    st, cos, fld = orc.quantize(w, S.BF16, g)
    assert st == 0
    x = (S.container_to_float(w, S.BF16) * g[:, None]).astype(np.float32).reshape(-1, 8)
    for v in range(x.shape[0]):
        z = orc.point_from_fields(fld[8 * v:8 * v + 8].astype(np.int32))
        p = z + 0.5 * cos[v]
        _, _, dmin = orc.e8_brute(x[v])
        d = float(np.sum((x[v].astype(np.float64) - p) ** 2))
        assert d <= dmin * (1 + 1e-6) + 1e-30


def test_quantize_row_selection_and_range_error(orc):
    w = S.iid_normal(8, 32, seed=4)
    ss = orc.row_sumsq(w, S.BF16)
    g = orc.gains(ss, 32, 0.5)
    st, cos_all, fld_all = orc.quantize(w, S.BF16, g)
    st2, cos_s, fld_s = orc.quantize(w, S.BF16, g, row_sel=[5, 2])
    assert st == 0 and st2 == 0
    vpr = 4
    assert np.array_equal(cos_s[:vpr], cos_all[5 * vpr:6 * vpr])
    assert np.array_equal(cos_s[vpr:], cos_all[2 * vpr:3 * vpr])
    assert np.array_equal(fld_s[:8 * vpr], fld_all[8 * 5 * vpr:8 * 6 * vpr])
    # a gain that puts a coordinate beyond the int16 field range is a range error
    g_big = g * np.float32(1e6)
    st3, _, _ = orc.quantize(w, S.BF16, g_big)
    assert st3 == orc.ERR_RANGE
