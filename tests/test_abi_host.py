"""CPU tests of libep.so: the library loads, exports every call declared in include/ep.h, and its
host-side logic (table normalisation, tile encoder, blob parser, rate estimate) matches the oracle
bit for bit.  No kernel is launched here."""

import os
import re

import numpy as np
import pytest

import ep_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ep():
    import entropy_coded_weight_ep_amd as ep

    if not os.path.exists(ep.lib_path()):
        pytest.skip("libep.so not built (run __graft_entry__.build())")
    ep.lib()
    return ep


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ep.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(ep_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(ep):
    names = declared_functions()
    assert len(names) >= 14
    lib = ep.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ep.ABI), "binding and header disagree"


def test_status_strings_and_defaults(ep):
    for st in range(11):
        assert ep.ep_status_string(st)
    cfg = ep.ep_config_default()
    assert cfg.tile_fields == 8192 and cfg.sample_rows == 256 and cfg.search_iters == 40
    assert cfg.refine == 0


def _hist_uint32(counts):
    return np.ascontiguousarray(counts.astype(np.uint32))


@pytest.mark.parametrize("seed", range(6))
def test_build_tables_matches_oracle(ep, orc, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    nv = int(g.integers(100, 5000))
    cos = (g.random(nv) < 0.3).astype(np.uint8)
    spread = [0.5, 2.0, 10.0, 60.0, 300.0, 1500.0][seed]
    fld = np.clip(np.rint(g.standard_t(3, nv * 8) * spread), -32767, 32767).astype(np.int16)
    counts = orc.histogram(cos, fld)
    st_o, lo_o, n_o, freq_o = orc.build_tables(counts)
    st, lo, n, freq = ep.ep_build_tables(_hist_uint32(counts))
    assert st == st_o
    if st == 0:
        assert np.array_equal(lo, lo_o) and np.array_equal(n, n_o)
        assert np.array_equal(freq, freq_o)


def test_build_tables_alphabet_error(ep, orc):
    counts = np.zeros((17, 65536), np.uint64)
    counts[0, 32768] = 10
    counts[1, 32768 - 3000:32768 + 1097] = 1          # 4097 distinct values
    st, *_ = ep.ep_build_tables(_hist_uint32(counts))
    assert st == ep.EP_ERR_ALPHABET
    assert orc.build_tables(counts)[0] == orc.ERR_ALPHABET


@pytest.mark.parametrize("nv,F", [(512, 4096), (5000, 4096), (40, 8192), (3000, 16384),
                                  (2048, 8192)])
def test_encode_tiles_matches_oracle(ep, orc, nv, F):
    g = np.random.Generator(np.random.PCG64(nv))
    cos = (g.random(nv) < 0.45).astype(np.uint8)
    fld = np.rint(g.standard_normal(nv * 8) * 3).astype(np.int16)
    counts = orc.histogram(cos, fld)
    st, lo, n, freq = orc.build_tables(counts)
    st_o, woff_o, states_o, words_o = orc.encode_tiles(cos, fld, F, 64, 12, lo, n, freq)
    st, woff, states, words = ep.ep_encode_tiles(cos, fld, F, ep.tables_struct(lo, n, freq))
    assert st == 0 and st_o == 0
    assert np.array_equal(woff, woff_o)
    assert np.array_equal(states, states_o)
    assert np.array_equal(words, words_o)


@pytest.mark.parametrize("key,shape", [(1, None), (2, (64, 1024)), (3, (64, 512)),
                                       ("5a", (16, 2048)), ("5b", (16, 2048))])
def test_blob_parse_on_oracle_blobs(ep, orc, key, shape):
    wl = S.WORKLOADS[key]
    R, Cc = shape or (wl["rows"], wl["cols"])
    w = S.workload_weights(key, R, Cc)
    st, blob, s = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
    assert st == 0
    st, info = ep.ep_blob_parse(blob)
    assert st == 0
    ref = orc.blob_fields(blob)
    assert (info.rows, info.cols, info.dtype, info.tile_fields, info.tiles) == \
        (ref["rows"], ref["cols"], ref["dtype"], ref["tile_fields"], ref["tiles"])
    assert info.scale == ref["s"] and info.payload_words == ref["payload_words"]
    assert info.actual_bpp == 8.0 * blob.size / (R * Cc)
    # the table records as written by the oracle
    p = 64
    for t in range(17):
        lo = int(blob[p:p + 4].view(np.int32)[0])
        n = int(blob[p + 4:p + 8].view(np.uint32)[0])
        assert info.lo[t] == lo and info.n[t] == n and info.table_off[t] == p
        if t == 0:
            assert info.coset_freq0 == int(blob[p + 8:p + 10].view(np.uint16)[0])
        p += (8 + 2 * n + 3) // 4 * 4


def test_blob_parse_rejects_corruption(ep, orc):
    w = S.workload_weights(1)
    st, blob, s = orc.compress(w, S.BF16, 3.5, 4096)
    assert ep.ep_blob_parse(blob)[0] == 0
    b = blob.copy(); b[0] = 0
    assert ep.ep_blob_parse(b)[0] == ep.EP_ERR_CORRUPT
    b = blob.copy(); b[4] = 7
    assert ep.ep_blob_parse(b)[0] == ep.EP_ERR_VERSION
    assert ep.ep_blob_parse(blob[:-16].copy())[0] == ep.EP_ERR_CORRUPT
    b = blob.copy(); b[64 + 8] ^= 1                       # coset frequencies no longer sum to M
    assert ep.ep_blob_parse(b)[0] == ep.EP_ERR_CORRUPT
    b = blob.copy(); b[6] = 9
    assert ep.ep_blob_parse(b)[0] == ep.EP_ERR_DTYPE


@pytest.mark.parametrize("alpha,tiny", [(1e-40, 1), (-1e-40, 1), (0.0, 0), (-0.0, 0),
                                         (2.0 ** -125, 0), (-(2.0 ** -125), 0),
                                         (np.nextafter(np.float32(2.0 ** -125), np.float32(0)), 1),
                                         (1.5, 0)])
def test_blob_parse_flags_tiny_scales(ep, orc, alpha, tiny):
    # a nonzero row scale below 2^-125 in magnitude has an inexact half: the parse flags it so
    # that the decoder scales such blobs without the fused multiply-add
    w = S.workload_weights(1)
    st, blob, s = orc.compress(w, S.BF16, 3.5, 4096)
    st, info = ep.ep_blob_parse(blob)
    assert st == 0 and info.tiny_scale == 0
    b = blob.copy()
    b[info.off_alpha + 4 * 7:info.off_alpha + 4 * 8] = np.array([alpha], np.float32).view(np.uint8)
    st, info2 = ep.ep_blob_parse(b)
    assert st == 0 and info2.tiny_scale == tiny


def _decoded_points(orc, blob, info):
    """(|p| of every decoded vector [NV, 8], |alpha| per row), from the oracle's decoded cosets
    and fields: z7 = 2 f7 + parity(f0..f6), p = z + c/2 (design page "EntroPack lattice
    compression", Lattice quantization and integer fields)."""
    st, _, cos, fld = orc.decompress(blob, want_fields=True)
    assert st == 0
    f = fld.reshape(-1, 8).astype(np.int64)
    z = f.copy()
    z[:, 7] = 2 * f[:, 7] + (f[:, :7].sum(axis=1) & 1)
    p = np.abs(z + 0.5 * cos[:, None])
    alpha = blob[info.off_alpha:info.off_alpha + 4 * info.rows].view(np.float32)
    return p, np.abs(alpha.astype(np.float64))


@pytest.mark.parametrize("key", [1, "5a", "5b"])
def test_blob_parse_bound_flag(ep, orc, key):
    # `bounded`: every value the tile decode writes lies within +-448.  The flag's bound on |p|
    # (from the field tables' value ranges) must cover every point the oracle's decode
    # reconstructs; the flag is set exactly when the largest |row scale| times that bound is at
    # most 448, which one row scale then crosses.
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, 32, 2048)
    st, blob, s = orc.compress(w, wl["dtype"], wl["target_bpp"], 4096)
    assert st == 0
    st, info = ep.ep_blob_parse(blob)
    assert st == 0
    p, alpha = _decoded_points(orc, blob, info)
    vpr = (info.cols + 7) // 8
    assert (alpha[np.arange(len(p)) // vpr][:, None] * p).max() <= 448.0
    assert info.bounded == 1
    mp = 0.0
    for t in range(1, 17):
        if info.n[t]:
            m = max(abs(info.lo[t]), abs(info.lo[t] + info.n[t] - 1))
            mp = max(mp, (2 * m + 1 if (t - 1) % 8 == 7 else m) + 0.5 * ((t - 1) // 8))
    assert p.max() <= mp
    a_max = np.float32(448.0 / mp)                  # the largest fp32 scale the bound admits
    while float(a_max) * mp > 448.0:
        a_max = np.nextafter(a_max, np.float32(0))
    assert alpha.max() <= a_max
    for a, want in ((a_max, 1), (np.nextafter(a_max, np.float32(1e9)), 0), (np.float32(1e3), 0),
                    (-a_max, 1), (np.float32(-1e3), 0)):
        b = blob.copy()
        b[info.off_alpha + 4 * 3:info.off_alpha + 4 * 4] = np.array([a], np.float32).view(np.uint8)
        st, info2 = ep.ep_blob_parse(b)
        assert st == 0 and info2.bounded == want, (a, want)


@pytest.mark.parametrize("s", [0.05, 0.3, 1.0, 4.0])
def test_estimate_matches_oracle(ep, orc, s):
    w = S.lognormal_rows(600, 512, seed=4)
    R, Cc = w.shape
    ns = 256
    sel = (np.arange(ns) * R) // ns
    ss = orc.row_sumsq(w, S.BF16)
    g = orc.gains(ss, Cc, s)
    st, cos, fld = orc.quantize(w, S.BF16, g, row_sel=sel)
    assert st == 0
    counts = orc.histogram(cos, fld)
    est = ep.ep_estimate_bpp(_hist_uint32(counts), R, Cc, ns, 4096)
    assert est == orc.estimate_bpp(w, S.BF16, 4096, s)


def test_compress_bound_covers_blobs(ep, orc):
    for key, shape in [(1, None), (3, (64, 512))]:
        wl = S.WORKLOADS[key]
        R, Cc = shape or (wl["rows"], wl["cols"])
        w = S.workload_weights(key, R, Cc)
        st, blob, s = orc.compress(w, wl["dtype"], 11.0, wl["tile_fields"])
        assert blob.size <= ep.ep_compress_bound(R, Cc, wl["tile_fields"])
    w = S.lognormal_rows(50, 1001, seed=7)              # a width that is not a multiple of 8
    st, blob, s = orc.compress(w, S.BF16, 11.0, 4096)
    assert st == 0 and blob.size <= ep.ep_compress_bound(50, 1001, 4096)
    st, info = ep.ep_blob_parse(blob)
    assert st == 0 and (info.rows, info.cols) == (50, 1001)
    assert info.tiles == (50 * 126 + 511) // 512
    with pytest.raises(ep.EPError):
        ep.ep_compress_bound(4, 0, 4096)


def test_encode_workspace_bytes(ep):
    # tables (17 x 65536 u32) + counts + one 9V-word stack per tile, each part 256-byte aligned
    up = lambda b: (b + 255) // 256 * 256
    for nv, F in [(1, 4096), (4773, 4096), (32768, 8192), (18441, 16384)]:
        V = F // 8
        T = (nv + V - 1) // V
        want = up(4 * 17 * 65536) + up(4 * T) + up(2 * 9 * V * T)
        assert ep.ep_encode_workspace_bytes(nv, F) == want
    assert ep.ep_encode_workspace_bytes(0, 4096) == 0
    assert ep.ep_encode_workspace_bytes(100, 1000) == 0


def test_rate_costs_match_oracle(ep, orc):
    assert np.array_equal(ep.ep_rate_costs(), orc.rate_costs())


@pytest.mark.parametrize("seed", range(6))
def test_refine_select_matches_oracle(ep, orc, seed):
    g = np.random.Generator(np.random.PCG64(900 + seed))
    rows, nc = int(g.integers(1, 300)), [1, 3, 5, 9, 3, 5][seed]
    Rq = g.integers(0, 1 << 30, (rows, nc)).astype(np.int64)
    D = g.uniform(0.0, 5.0, (rows, nc))
    if nc > 1:
        D[g.random((rows, nc)) < 0.1] = np.inf          # candidates not offered
        D[:, (nc - 1) // 2] = g.uniform(0.0, 5.0, rows)  # the middle one always is
    lo, hi = int(Rq.min(axis=1).sum()), int(Rq.max(axis=1).sum())
    for budget in (lo - 1, lo, (lo + hi) // 2, hi, hi + 1, 0):
        lam, sel = ep.ep_refine_select(D, Rq, budget)
        lam_o, sel_o = orc.refine_select(D, Rq, budget)
        assert np.float64(lam).view(np.uint64) == np.float64(lam_o).view(np.uint64)
        assert np.array_equal(sel, sel_o)


def test_encoder_quotient_estimate_bound():
    """The device tile encoder divides x by the frequency f (1..4096) with an fp32 estimate
    (x rounded to fp32, times the hardware reciprocal, which is within 1 ulp of 1/f), truncated,
    then corrected by a single integer step.  That is exact only if the truncated estimate is
    never more than 1 away from floor(x / f) while x < f * 2^20: swept here for every f, with
    the reciprocal rounded correctly and off by one ulp either way, at the largest quotients,
    around every multiple of f there, and at random ones."""
    f = np.arange(1, 4097, dtype=np.int64)
    rc0 = (np.float32(1.0) / f.astype(np.float32)).astype(np.float32)
    worst = 0
    rng = np.random.default_rng(5)
    ff = rng.integers(1, 4097, 500_000)
    xr = (rng.random(500_000) * ff * (1 << 20)).astype(np.int64)
    for rc in (rc0, np.nextafter(rc0, np.float32(0)), np.nextafter(rc0, np.float32(np.inf))):
        for k in list(range((1 << 20) - 16, 1 << 20)) + [0, 1, 2, 65535, 65536]:
            for d in (-1, 0, 1):
                x = k * f + d
                ok = (x >= 0) & (x < f * (1 << 20))
                if not ok.any():
                    continue
                q = (x[ok].astype(np.float32) * rc[ok]).astype(np.float32)
                est = np.floor(q.astype(np.float64)).astype(np.int64)
                worst = max(worst, int(np.abs(est - x[ok] // f[ok]).max()))
        q = (xr.astype(np.float32) * rc[ff - 1]).astype(np.float32)
        est = np.floor(q.astype(np.float64)).astype(np.int64)
        worst = max(worst, int(np.abs(est - xr // ff).max()))
    assert worst <= 1


def test_blob_parse_exception_list(ep, orc):
    """The parser reads a version-1.1 blob's exception list where the oracle wrote it, and rejects
    a list out of order, a vector past the end, and a count the version does not allow."""
    w = S.student_t_outliers(512, 1024, seed=11, nu=2.0, scale=0.02)
    st, blob, _ = orc.compress(w, S.FP16, 3.0, 8192, force_s=1.0 / 1000.0)
    assert st == 0
    X = orc.blob_exceptions(blob)
    assert X >= 2
    st, info = ep.ep_blob_parse(blob)
    assert st == 0 and info.n_exceptions == X
    o, of = info.off_exceptions, info.off_exception_fields
    assert o % 16 == 0 and of % 16 == 0 and of + 16 * X == blob.size
    assert of == o + (4 * X + 15) // 16 * 16
    nv = info.rows * ((info.cols + 7) // 8)
    idx = blob[o: o + 4 * X].view(np.uint32)
    assert np.all(np.diff(idx & 0x7FFFFFFF) > 0) and int(idx[-1] & 0x7FFFFFFF) < nv
    bad = blob.copy()
    bi = bad[o: o + 4 * X].view(np.uint32)
    bi[0], bi[1] = idx[1], idx[0]
    assert ep.ep_blob_parse(bad)[0] == ep.EP_ERR_CORRUPT
    bad = blob.copy()
    bad[o + 4 * (X - 1): o + 4 * X].view(np.uint32)[0] = nv
    assert ep.ep_blob_parse(bad)[0] == ep.EP_ERR_CORRUPT
    bad = blob.copy()
    bad[5] = 0
    assert ep.ep_blob_parse(bad)[0] == ep.EP_ERR_CORRUPT
    bad = blob.copy()
    bad[5] = 2
    assert ep.ep_blob_parse(bad)[0] == ep.EP_ERR_VERSION
    # a blob without escapes is version 1.0 with no list
    st, blob0, _ = orc.compress(S.workload_weights(2, 64, 1024, 0), S.BF16, 4.0, 8192)
    st, info0 = ep.ep_blob_parse(blob0)
    assert st == 0 and info0.n_exceptions == 0 and info0.off_exceptions == 0


def test_blob_parse_rejects_shapes_that_would_overflow(ep, orc):
    """Crafted headers whose vector count rows * ceil(cols / 8) is past 2^31 (or past int64) are
    corrupt; the check runs before the product is formed."""
    st, blob, _ = orc.compress(S.workload_weights(1), S.BF16, 3.5, 4096)
    assert ep.ep_blob_parse(blob)[0] == 0
    for rows, cols in [(1 << 40, 1 << 40), (1 << 31, 8), (1 << 28, 64), ((1 << 31) - 1, 16)]:
        b = blob.copy()
        b[8:16] = np.array([rows], np.uint64).view(np.uint8)
        b[16:24] = np.array([cols], np.uint64).view(np.uint8)
        assert ep.ep_blob_parse(b)[0] == ep.EP_ERR_CORRUPT, (rows, cols)
    # entry points that take shapes from the caller refuse them the same way
    assert ep.ep_compress_workspace_bytes(1 << 40, 1 << 40) == 0
    with pytest.raises(Exception):
        ep.ep_compress_bound(1 << 31, 8, 4096)


# ------------------------------------------------------------------------------------------
# 128 states per tile (two per wavefront lane) and the rate-search settings, on the host
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("nv,F", [(512, 4096), (5000, 4096), (100, 8192), (3000, 16384),
                                  (2048, 8192)])
def test_encode_tiles_128_lanes_matches_oracle(ep, orc, nv, F):
    g = np.random.Generator(np.random.PCG64(nv + 7))
    cos = (g.random(nv) < 0.45).astype(np.uint8)
    fld = np.rint(g.standard_normal(nv * 8) * 3).astype(np.int16)
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    st_o, woff_o, states_o, words_o = orc.encode_tiles(cos, fld, F, 128, 12, lo, n, freq)
    st, woff, states, words = ep.ep_encode_tiles(cos, fld, F, ep.tables_struct(lo, n, freq),
                                                 lanes=128)
    assert st == 0 and st_o == 0
    assert np.array_equal(woff, woff_o)
    assert np.array_equal(states, states_o)
    assert np.array_equal(words, words_o)


def test_encode_tiles_rejects_other_lane_counts(ep, orc):
    cos = np.zeros(512, np.uint8)
    fld = np.zeros(512 * 8, np.int16)
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    tab = ep.tables_struct(lo, n, freq)
    for lanes in (32, 96, 256):
        assert ep.ep_encode_tiles(cos, fld, 4096, tab, lanes=lanes)[0] == ep.EP_ERR_ARG
    # a tile of 64 vectors cannot hold 128 states' worth of vectors
    assert ep.ep_encode_tiles(cos, fld, 512, tab, lanes=128)[0] == ep.EP_ERR_ARG


@pytest.mark.parametrize("key,shape", [(1, None), (2, (64, 1024)), (3, (64, 512)),
                                       ("5b", (16, 2048))])
def test_blob_parse_128_lanes(ep, orc, key, shape):
    wl = S.WORKLOADS[key]
    R, Cc = shape or (wl["rows"], wl["cols"])
    w = S.workload_weights(key, R, Cc)
    st, blob, s = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"], lanes=128)
    assert st == 0
    st, info = ep.ep_blob_parse(blob)
    assert st == 0 and info.lanes == 128
    ref = orc.blob_fields(blob)
    T = ref["tiles"]
    assert info.off_words - info.off_states == (4 * 128 * T + 15) // 16 * 16
    assert info.payload_words == ref["payload_words"] and info.bytes == blob.size


@pytest.mark.parametrize("lanes", [64, 128])
@pytest.mark.parametrize("ns", [40, 256, 600])
def test_estimate_matches_oracle_at_each_setting(ep, orc, lanes, ns):
    w = S.lognormal_rows(600, 512, seed=4)
    R, Cc = w.shape
    s = 0.3
    sel = (np.arange(min(ns, R)) * R) // min(ns, R)
    g = orc.gains(orc.row_sumsq(w, S.BF16), Cc, s)
    st, cos, fld = orc.quantize(w, S.BF16, g, row_sel=sel)
    assert st == 0
    est = ep.ep_estimate_bpp(_hist_uint32(orc.histogram(cos, fld)), R, Cc, sel.size, 8192,
                             lanes=lanes)
    assert est == orc.estimate_bpp(w, S.BF16, 8192, s, lanes=lanes, sample_rows=ns)
