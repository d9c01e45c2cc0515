"""Oracle pins for escapes: a field table that would hold more than 2^12 distinct values keeps the
2^12 most frequent, the tiles code every other value as the table's substitute, and the blob's
exception list restores the true vectors.

What fixes the oracle here, independently of its coding path:
  - the kept set against properties any correct ranking has (exactly M kept, every kept count
    at least every dropped one, lower values first among equal counts at the boundary);
  - the tables built from the kept counts alone (nonzero exactly on the kept values, sum M);
  - lossless coding: a blob with escapes decodes to the direct reconstruction of the quantised
    vectors (fields from the quantiser, alpha from the LS terms, y = fp32(alpha * h / 2)), so a
    dropped or misplaced exception or a wrong coset bit fails it (the substitute itself only
    decides which kept symbol stands in; the library's blob must match the oracle's byte for
    byte, which fixes it);
  - the exception list against a numpy scan for vectors with a field their table lacks.
"""
import numpy as np
import pytest

import ep_synth as S
import oracle

M = 4096


def _escape_tensor(seed=11):
    # Student-t(2) rows at s = 1/1000: a few field tables exceed 4096 distinct values
    return S.student_t_outliers(512, 1024, seed=seed, nu=2.0, scale=0.02)


def test_escape_keep_properties():
    g = np.random.default_rng(5)
    c = np.zeros(oracle.NBINS, np.uint64)
    bins = g.choice(oracle.NBINS, 6000, replace=False)
    c[bins] = g.integers(1, 40, bins.size).astype(np.uint64)   # many equal counts
    kept = oracle.escape_keep(c)
    assert kept.sum() == M and np.all(c[kept] > 0)
    dropped = (c > 0) & ~kept
    assert dropped.sum() == 6000 - M
    assert c[kept].min() >= c[dropped].max()
    edge = c[kept].min()
    if c[dropped].max() == edge:                  # ties at the boundary: lower values kept
        kb = np.flatnonzero(kept & (c == edge))
        db = np.flatnonzero(dropped & (c == edge))
        assert kb.max() < db.min()
    # at most M distinct values: all kept
    c2 = np.zeros(oracle.NBINS, np.uint64)
    c2[bins[:M]] = 3
    assert np.array_equal(oracle.escape_keep(c2), c2 > 0)


def test_escape_tables():
    g = np.random.default_rng(6)
    counts = np.zeros((oracle.NTABLES, oracle.NBINS), np.uint64)
    counts[0, 32768] = 900
    counts[0, 32769] = 100
    for t in range(1, oracle.NTABLES):
        d = 5000 if t in (3, 12) else 300        # two tables overflow
        b = 32768 + g.choice(np.arange(-6000, 6000), d, replace=False)
        counts[t, b] = g.integers(1, 1000, d).astype(np.uint64)
    st, lo, n, freq = oracle.build_tables_escapes(counts)
    assert st == 0
    st0, lo0, n0, freq0 = oracle.build_tables(counts)
    assert st0 == oracle.ERR_ALPHABET
    for t in range(oracle.NTABLES):
        f = freq[t, : n[t]].astype(np.int64)
        assert f.sum() == M
        present = np.zeros(oracle.NBINS, bool)
        present[lo[t] + 32768: lo[t] + 32768 + n[t]] = f > 0
        if t in (3, 12):
            assert np.array_equal(present, oracle.escape_keep(counts[t]))
        else:
            assert np.array_equal(present, counts[t] > 0)
            one = counts.copy()
            one[3] = 0
            one[12] = 0
            st1, lo1, n1, freq1 = oracle.build_tables(one)
            assert st1 == 0 and lo1[t] == lo[t] and n1[t] == n[t]
            assert np.array_equal(freq1[t, : n[t]], freq[t, : n[t]])
    # the substitute is the most probable value, the lowest on ties
    for t in (3, 12):
        f = freq[t, : n[t]]
        assert oracle.substitute(lo[t], n[t], f) == lo[t] + int(np.argmax(f))


def _direct_reconstruction(w, dt, s):
    """Quantise at s and reconstruct without any coding: the values a lossless blob must give."""
    R, C = w.shape
    gains = oracle.gains(oracle.row_sumsq(w, dt), C, s)
    st, cos, fld = oracle.quantize(w, dt, gains)
    assert st == 0
    num, den4 = oracle.row_lsq(w, dt, cos, fld)
    alpha = np.array([oracle.alpha(a, b) for a, b in zip(num, den4)], np.float32)
    vpr = (C + 7) // 8
    f = fld.reshape(-1, 8).astype(np.int64)
    z = f.copy()
    z[:, 7] = 2 * f[:, 7] + (f[:, :7].sum(axis=1) & 1)       # parity of the first seven
    h = 2 * z + cos.astype(np.int64)[:, None]
    p = h.astype(np.float32) * np.float32(0.5)
    y = (np.repeat(alpha, vpr)[:, None] * p).astype(np.float32).reshape(R, vpr * 8)[:, :C]
    return S.cast_container(np.ascontiguousarray(y), dt), cos, fld


@pytest.mark.parametrize("F", [4096, 8192, 16384])
def test_escape_round_trip(F):
    w = _escape_tensor()
    s = 1.0 / 1000.0
    st, blob, _ = oracle.compress(w, S.FP16, 3.0, F, force_s=s)
    assert st == 0
    X = oracle.blob_exceptions(blob)
    assert X > 0 and blob[4] == 1 and blob[5] == 1
    assert int(blob[60:64].view(np.uint32)[0]) == X
    st, out, cos, fld = oracle.decompress(blob, want_fields=True)
    assert st == 0
    ref, qcos, qfld = _direct_reconstruction(w, S.FP16, s)
    assert np.array_equal(cos, qcos) and np.array_equal(fld, qfld)
    assert np.array_equal(out, ref)


def test_escape_list_matches_scan():
    w = _escape_tensor()
    s = 1.0 / 1000.0
    _, qcos, qfld = _direct_reconstruction(w, S.FP16, s)
    counts = oracle.histogram(qcos, qfld)
    st, lo, n, freq = oracle.build_tables_escapes(counts)
    assert st == 0
    idx, xf = oracle.exceptions(qcos, qfld, lo, n, freq)
    f = qfld.reshape(-1, 8).astype(np.int64)
    c = qcos.astype(np.int64)
    lacking = np.zeros(f.shape[0], bool)
    for k in range(8):
        t = 1 + 8 * c + k
        q = f[:, k] - lo[t]
        inside = (q >= 0) & (q < n[t])
        fq = np.zeros(f.shape[0], np.int64)
        fq[inside] = freq[t[inside], q[inside]]
        lacking |= fq == 0
    v = np.flatnonzero(lacking)
    assert v.size == idx.size > 0
    assert np.array_equal(idx & 0x7FFFFFFF, v.astype(np.uint32))
    assert np.array_equal(idx >> 31, qcos[v].astype(np.uint32))
    assert np.array_equal(xf, qfld.reshape(-1, 8)[v])
    # and the blob carries exactly this list
    st, blob, _ = oracle.compress(w, S.FP16, 3.0, 8192, force_s=s)
    assert st == 0 and oracle.blob_exceptions(blob) == idx.size


def test_escape_tile_ranges():
    """Decoding a tile range patches the escaped vectors inside it and writes nothing outside."""
    w = _escape_tensor()
    st, blob, _ = oracle.compress(w, S.FP16, 3.0, 4096, force_s=1.0 / 1000.0)
    assert st == 0
    st, full, _, _ = oracle.decompress(blob)
    assert st == 0
    T = oracle.blob_fields(blob)["tiles"]
    t0, t1 = T // 3, 2 * T // 3
    st, part, _, _ = oracle.decompress(blob, t0, t1)
    assert st == 0
    flat, pflat = full.reshape(-1), part.reshape(-1)
    e0, e1 = t0 * 4096, t1 * 4096
    assert np.array_equal(pflat[e0:e1], flat[e0:e1])
    assert not pflat[:e0].any() and not pflat[e1:].any()


def test_no_escape_blob_is_version_1_0():
    w = S.workload_weights(2, 64, 1024, 0)
    st, blob, _ = oracle.compress(w, S.BF16, 4.0, 8192)
    assert st == 0 and blob[4] == 1 and blob[5] == 0 and not blob[60:64].any()
    assert oracle.blob_exceptions(blob) == 0


def _status(blob):
    return oracle.lib().or_decompress(oracle._p(blob), blob.size, 0, -1, None, None, None)


def test_escape_blob_corruption():
    w = _escape_tensor()
    st, blob, _ = oracle.compress(w, S.FP16, 3.0, 8192, force_s=1.0 / 1000.0)
    assert st == 0
    X = oracle.blob_exceptions(blob)
    assert X >= 2
    info = oracle.blob_fields(blob)
    o_x = blob.size - 16 * X - ((4 * X + 15) // 16 * 16)
    idx = blob[o_x: o_x + 4 * X].view(np.uint32)
    bad = blob.copy()                               # exception list out of order
    bi = bad[o_x: o_x + 4 * X].view(np.uint32)
    bi[0], bi[1] = idx[1], idx[0]
    assert _status(bad) == oracle.ERR_CORRUPT
    bad = blob.copy()                               # a vector past the end
    bad[o_x + 4 * (X - 1): o_x + 4 * X].view(np.uint32)[0] = 0x7FFFFFFF
    assert _status(bad) == oracle.ERR_CORRUPT
    bad = blob.copy()                               # count disagrees with the version
    bad[5] = 0
    assert _status(bad) == oracle.ERR_CORRUPT
    bad = blob.copy()                               # unknown minor version
    bad[5] = 2
    assert _status(bad) == oracle.ERR_VERSION
    assert info["tiles"] > 0
