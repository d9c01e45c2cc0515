"""Pins for the oracle's per-row rate-distortion refinement (EntroPack design page, "Rate
selection and refinement": several resolutions per row, handed out under an estimated storage
budget, alternating with updates of the shared model; off by default).

What pins it, apart from its own formulas:
- the code lengths at powers of two are exact bit counts;
- the per-row rates add up to the per-bin sum over the histogram that built the model, and a
  value the model lacks costs exactly P + 1 bits;
- the Lagrangian selection, checked by brute force on small cases: it minimises D + lambda R over
  every combination, no combination with a lower or equal total rate has a lower total
  distortion, the budget holds when it can, and a slightly smaller lambda breaks it;
- one candidate reduces the refinement to the plain path (byte-identical blobs);
- on rows with very different scales the refinement lowers the relative L2 error at the same
  target rate.
"""

import itertools

import numpy as np
import pytest

import ep_synth as S

ONE = 65536


def test_rate_costs_closed_forms(orc):
    c = orc.rate_costs()
    assert c[0] == 13 * ONE                       # a value absent from the model: P + 1 bits
    for e in range(13):                           # f = 2^e costs exactly 12 - e bits
        assert c[1 << e] == (12 - e) * ONE
    assert np.all(np.diff(c[1:].astype(np.int64)) <= 0)


def _model(orc, cos, fld):
    counts = orc.histogram(cos, fld)
    st, lo, n, freq = orc.build_tables(counts)
    assert st == 0
    return counts, lo, n, freq


def test_row_rates_add_up_to_the_histogram_sum(orc):
    w = S.lognormal_rows(40, 256, seed=41)
    g = orc.gains(orc.row_sumsq(w, S.BF16), 256, 0.2)
    st, cos, fld = orc.quantize(w, S.BF16, g)
    assert st == 0
    counts, lo, n, freq = _model(orc, cos, fld)
    cost = orc.rate_costs()
    rates = orc.row_rates(cos, fld, 40, 256, lo, n, freq, cost)
    per_bin = 0
    for t in range(17):
        for i in range(int(n[t])):
            k = int(counts[t, int(lo[t]) + 32768 + i])
            if k:
                per_bin += k * int(cost[int(freq[t, i])])
    assert int(rates.sum()) == per_bin
    # the fixed-point sum is within half a unit per symbol of the exact code length
    exact = sum(int(counts[t, int(lo[t]) + 32768 + i]) * (12 - np.log2(freq[t, i]))
                for t in range(17) for i in range(int(n[t])) if counts[t, int(lo[t]) + 32768 + i])
    assert abs(per_bin / ONE - exact) <= 40 * 32 * 9 / (2 * ONE) + 1e-9


def test_row_rate_of_a_value_outside_the_model(orc):
    w = S.lognormal_rows(8, 64, seed=42)
    g = orc.gains(orc.row_sumsq(w, S.BF16), 64, 0.3)
    st, cos, fld = orc.quantize(w, S.BF16, g)
    counts, lo, n, freq = _model(orc, cos, fld)
    cost = orc.rate_costs()
    base = orc.row_rates(cos, fld, 8, 64, lo, n, freq, cost)
    v, k = 10, 2                                  # row 1, vector 2 of that row, field 2
    t = 1 + 8 * int(cos[v]) + k
    old = int(fld[8 * v + k])
    f_old = int(freq[t, old - int(lo[t])])
    bad = fld.copy()
    bad[8 * v + k] = int(lo[t]) + int(n[t]) + 3   # outside the table's span
    rates = orc.row_rates(cos, bad, 8, 64, lo, n, freq, cost)
    assert rates[1] - base[1] == 13 * ONE - int(cost[f_old])
    assert np.array_equal(np.delete(rates, 1), np.delete(base, 1))


def _pick(D, Rq, lam):
    J = D + lam * (Rq.astype(np.float64) / ONE)
    return np.argmin(J, axis=1)


@pytest.mark.parametrize("seed", range(8))
def test_refine_select_brute_force(orc, seed):
    g = np.random.Generator(np.random.PCG64(500 + seed))
    rows, nc = 5, 3
    # finer candidates (low k): more bits, less distortion, with noise
    Rq = (np.sort(g.integers(1000, 40000, (rows, nc)), axis=1)[:, ::-1] * 16).astype(np.int64)
    D = np.sort(g.uniform(0.01, 2.0, (rows, nc)), axis=1)
    lo_tot, hi_tot = int(Rq.min(axis=1).sum()), int(Rq.max(axis=1).sum())
    for budget in (lo_tot - 5, lo_tot + (hi_tot - lo_tot) // 3, lo_tot + 2 * (hi_tot - lo_tot) // 3,
                   hi_tot + 5):
        lam, sel = orc.refine_select(D, Rq, budget)
        idx = np.arange(rows)
        tot = int(Rq[idx, sel].sum())
        dsum = float(D[idx, sel].sum())
        if budget >= lo_tot:
            assert tot <= budget
        if lam == 0.0:
            assert np.array_equal(sel, np.argmin(D, axis=1))
        # Lagrangian optimality and no better selection at a lower or equal rate
        j_sel = dsum + lam * tot / ONE
        for combo in itertools.product(range(nc), repeat=rows):
            c = np.array(combo)
            r = int(Rq[idx, c].sum())
            d = float(D[idx, c].sum())
            assert j_sel <= d + lam * r / ONE + 1e-9 * (1 + abs(j_sel))
            if r <= tot:
                assert dsum <= d + 1e-12
        # the smallest such lambda: a slightly smaller one breaks the budget
        if 0.0 < lam < 2.0 ** 60 and lam > 2.0 ** -59:
            s2 = _pick(D, Rq, lam * (1 - 1e-9))
            assert int(Rq[idx, s2].sum()) > budget


@pytest.mark.parametrize("key,shape", [(1, None), (2, (64, 512)), ("5a", (16, 1024))])
def test_refine_with_one_candidate_is_the_plain_path(orc, key, shape):
    wl = S.WORKLOADS[key]
    R, Cc = shape or (wl["rows"], wl["cols"])
    w = S.workload_weights(key, R, Cc)
    st0, b0, s0 = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
    st1, b1, s1 = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"], refine=1)
    assert st0 == st1 == 0 and s0 == s1
    assert np.array_equal(b0, b1)


def test_refine_lowers_error_on_rows_of_different_scale(orc):
    w = S.lognormal_rows(128, 512, seed=43, sigma=0.8)
    ref = S.container_to_float(w, S.BF16).astype(np.float64)
    out = {}
    for nc in (0, 5):
        st, blob, s = orc.compress(w, S.BF16, 3.0, 4096, refine=nc)
        assert st == 0
        st, dec, _, _ = orc.decompress(blob)
        assert st == 0
        rec = S.container_to_float(dec, S.BF16).astype(np.float64)
        out[nc] = (np.linalg.norm(rec - ref) / np.linalg.norm(ref), 8.0 * blob.size / w.size)
    (e0, b0), (e5, b5) = out[0], out[5]
    assert e5 < 0.95 * e0, out
    assert abs(b5 - 3.0) < 0.3, out


def test_refine_arguments(orc):
    w = S.iid_normal(16, 64, seed=1)
    for bad in (-1, 2, 4, 11):
        assert orc.compress(w, S.BF16, 3.0, 4096, refine=bad)[0] == orc.ERR_ARG
    assert orc.compress(w, S.BF16, 3.0, 4096, refine=3)[0] == 0
