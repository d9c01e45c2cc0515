"""Pins for the oracle's lane count and rate-search settings.

Lanes (design page "EntroPack lattice compression", *Encoding and reconstruction*: rANS in
independently decodable tiles).  A tile of V vectors is coded by K interleaved states, K = 64
(one per wavefront lane) or K = 128 (two per lane); state k owns the tile's vectors k, k + K, ...
and words are consumed phase by phase, vector index by vector index, state by state.  K is a
parameter of the same coder, so the pins are those of K = 64 at K = 128: the round trip is exact
(the coder is lossless), every state ends back at 2^16, the stream's size sits within the ideal
code length +- 16 bits per final state, corruption is caught, and a blob coded with 128 lanes
decodes to the same tensor, bit for bit, as one coded with 64 at the same scale.

Rate-search settings (*Rate selection and refinement*: the scale is searched on sampled rows;
*Usage*: search settings are part of the configuration).  sample_rows = n picks rows
floor(i R / n); the estimate of the whole tensor from that sample must equal the estimate of the
n-row matrix of exactly those rows (all of its rows sampled), scaled by R / n, once each side's
metadata is taken out in closed form.  search_iters = k: the returned scale meets the target and
the scale one final bisection step finer (log2 s - 32 / 2^k) does not.
"""

import numpy as np
import pytest

import ep_synth as S


def _random_fields(nv, seed, spread=3.0, heavy=False):
    g = np.random.Generator(np.random.PCG64(seed))
    cos = (g.random(nv) < 0.4).astype(np.uint8)
    if heavy:
        fld = np.rint(g.standard_t(2.5, nv * 8) * spread).clip(-3000, 3000).astype(np.int16)
    else:
        fld = np.rint(g.standard_normal(nv * 8) * spread).astype(np.int16)
    return cos, fld


def _ideal_bits(orc, cos, fld, lo, n, freq):
    counts = orc.histogram(cos, fld)
    bits = 0.0
    for t in range(17):
        for q in range(int(n[t])):
            c = counts[t, lo[t] + 32768 + q]
            if c:
                bits += float(c) * (12 - np.log2(float(freq[t, q])))
    return bits


@pytest.mark.parametrize("nv,F,spread,heavy", [
    (512, 4096, 3.0, False),         # exactly one tile
    (5000, 4096, 3.0, False),        # ragged last tile
    (100, 4096, 1.0, False),         # fewer vectors than states
    (2500, 8192, 40.0, True),        # heavy tails, large alphabets
    (6000, 16384, 8.0, False),
])
def test_rans_128_lanes_roundtrip_and_size(orc, nv, F, spread, heavy):
    cos, fld = _random_fields(nv, seed=3 * nv + F, spread=spread, heavy=heavy)
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    assert st == 0
    st, woff, states, words = orc.encode_tiles(cos, fld, F, 128, 12, lo, n, freq)
    assert st == 0
    T = woff.size - 1
    assert states.size == 128 * T
    st, cos2, fld2 = orc.decode_tiles(woff, states, words, nv, F, 128, 12, lo, n, freq)
    assert st == 0                      # every state back at 2^16, every word consumed
    assert np.array_equal(cos2, cos) and np.array_equal(fld2, fld)
    cost = _ideal_bits(orc, cos, fld, lo, n, freq)
    payload = 16.0 * woff[-1]
    assert payload >= cost - 16 * 128 * T - 1e-6
    assert payload <= cost * 1.01 + 16 * 128 * T
    # the information the coder keeps: words plus each final state's excess over 2^16
    kept = payload + float(np.sum(np.log2(states.astype(np.float64)) - 16.0))
    assert abs(kept - cost) <= 8.0 + 9 * nv * 2.0 ** -12


def test_rans_128_lanes_word_order_differs_from_64(orc):
    """Same symbols, two lane counts: both decode exactly; the streams differ (the states own
    different vectors), and each decoder rejects the other's stream."""
    nv = 2048
    cos, fld = _random_fields(nv, seed=11)
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    st, w64, s64, d64 = orc.encode_tiles(cos, fld, 8192, 64, 12, lo, n, freq)
    st2, w128, s128, d128 = orc.encode_tiles(cos, fld, 8192, 128, 12, lo, n, freq)
    assert st == 0 and st2 == 0
    assert not (w64.size == w128.size and np.array_equal(d64[:min(d64.size, d128.size)],
                                                         d128[:min(d64.size, d128.size)]))
    st, c, f = orc.decode_tiles(w128, s128, d128, nv, 8192, 128, 12, lo, n, freq)
    assert st == 0 and np.array_equal(f, fld)
    # a 64-lane decoder reading the first 64 of the 128 states cannot end every state at 2^16
    s_cut = s128.reshape(-1, 128)[:, :64].reshape(-1).copy()
    st, _, _ = orc.decode_tiles(w128, s_cut, d128, nv, 8192, 64, 12, lo, n, freq)
    assert st == orc.ERR_CORRUPT


def test_rans_128_lanes_corruption_is_detected(orc):
    cos, fld = _random_fields(4096, seed=5)
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    st, woff, states, words = orc.encode_tiles(cos, fld, 4096, 128, 12, lo, n, freq)
    bad = states.copy()
    bad[100] ^= 0x5A5A                                  # a state of the second half
    st, _, _ = orc.decode_tiles(woff, bad, words, 4096, 4096, 128, 12, lo, n, freq)
    assert st == orc.ERR_CORRUPT
    short = woff.copy()
    short[1] -= 1
    st, _, _ = orc.decode_tiles(short, states, words, 4096, 4096, 128, 12, lo, n, freq, 0, 1)
    assert st == orc.ERR_CORRUPT


def _pad16(n):
    return (n + 15) // 16 * 16


def _table_bytes(ns):
    return _pad16(sum((8 + 2 * int(x) + 3) // 4 * 4 for x in ns))


@pytest.mark.parametrize("key,R,C,dt,F", [(2, 96, 512, S.BF16, 8192), (1, 256, 256, S.BF16, 4096),
                                          (3, 64, 1000, S.FP16, 16384)])
def test_blob_with_128_lanes(orc, key, R, C, dt, F):
    """Same forced scale: the 128-lane blob decodes to the 64-lane blob's tensor bit for bit, its
    size is the closed-form section sum with 128 states per tile, and its header says K = 128."""
    w = S.workload_weights(key, R, C)
    s = 0.3
    st, b64, _ = orc.compress(w, dt, 1.0, F, force_s=s)
    st2, b128, _ = orc.compress(w, dt, 1.0, F, force_s=s, lanes=128)
    assert st == 0 and st2 == 0
    assert int(b128[28:32].view(np.uint32)[0]) == 128
    assert int(b64[28:32].view(np.uint32)[0]) == 64
    i64, i128 = orc.blob_fields(b64), orc.blob_fields(b128)
    T = i128["tiles"]
    assert i64["table_bytes"] == i128["table_bytes"]
    size = (64 + i128["table_bytes"] + _pad16(4 * R) + _pad16(4 * (T + 1)) + _pad16(4 * 128 * T)
            + _pad16(2 * i128["payload_words"]))
    assert b128.size == size
    st, o64, c64, f64 = orc.decompress(b64, want_fields=True)
    st2, o128, c128, f128 = orc.decompress(b128, want_fields=True)
    assert st == 0 and st2 == 0
    assert np.array_equal(o64, o128)
    assert np.array_equal(c64, c128) and np.array_equal(f64, f128)
    # tile-range decode of a 128-lane blob
    if T > 1:
        out = np.zeros_like(o128)
        st = orc.lib().or_decompress(orc._p(b128), b128.size, 1, T, orc._p(out), None, None)
        assert st == 0
        V = F // 8
        first = min(V * 8, R * C)
        assert np.array_equal(out.reshape(-1)[first:], o128.reshape(-1)[first:])


def test_unsupported_lane_counts_are_refused(orc):
    w = S.workload_weights(1)
    for lanes in (32, 96, 256):
        st, _, _ = orc.compress(w, S.BF16, 3.5, 4096, lanes=lanes)
        assert st == orc.ERR_ARG
    # 128 lanes need a tile of a multiple of 128 vectors
    st, _, _ = orc.compress(w, S.BF16, 3.5, 512, lanes=128)
    assert st == orc.ERR_ARG
    # a blob header claiming another lane count is refused by the parser
    st, blob, _ = orc.compress(w, S.BF16, 3.5, 4096)
    bad = blob.copy()
    bad[28:32] = np.array([32], np.uint32).view(np.uint8)
    with pytest.raises(ValueError):
        orc.blob_fields(bad)


@pytest.mark.parametrize("lanes", [64, 128])
def test_estimate_matches_the_coded_information_at_each_lane_count(orc, lanes):
    """With every row sampled the estimate's payload term is the ideal code length of what the
    encoder codes; words plus the final states' excess over 2^16 keep exactly that (up to the
    coder's floor losses).  The metadata counts `lanes` states per tile."""
    R, C, F = 64, 1024, 8192
    w = S.workload_weights(2, R, C)
    for s in (0.1, 0.5):
        est = orc.estimate_bpp(w, S.BF16, F, s, lanes=lanes)
        st, blob, _ = orc.compress(w, S.BF16, 1.0, F, force_s=s, lanes=lanes)
        assert st == 0
        info = orc.blob_fields(blob)
        T, W = info["tiles"], info["payload_words"]
        off_states = 64 + info["table_bytes"] + _pad16(4 * R) + _pad16(4 * (T + 1))
        meta = off_states + _pad16(4 * lanes * T)
        x = blob[off_states:off_states + 4 * lanes * T].view(np.uint32).astype(np.float64)
        coded = 16.0 * W + float(np.sum(np.log2(x) - 16.0))
        ideal = est * R * C - 8.0 * meta
        assert abs(ideal - coded) <= 8.0 + 9 * R * (C // 8) * 2.0 ** -12


@pytest.mark.parametrize("R,n", [(300, 256), (1000, 64), (97, 40), (50, 50), (50, 80)])
def test_sampled_rows_estimate(orc, R, n):
    C, F, s = 512, 8192, 0.25
    w = S.workload_weights(2, R, C)
    sel = (np.arange(min(n, R)) * R) // min(n, R)
    sub = np.ascontiguousarray(w[sel])
    ns = sub.shape[0]
    st, cos, fld = orc.quantize(sub, S.BF16, orc.gains(orc.row_sumsq(sub, S.BF16), C, s))
    assert st == 0
    st, lo, nn, freq = orc.build_tables(orc.histogram(cos, fld))
    tb = _table_bytes(nn)

    def meta(rows):
        T = (rows * C // 8 + F // 8 - 1) // (F // 8)
        return 64 + tb + _pad16(4 * rows) + _pad16(4 * (T + 1)) + _pad16(4 * 64 * T)

    whole = orc.estimate_bpp(w, S.BF16, F, s, sample_rows=n)
    part = orc.estimate_bpp(sub, S.BF16, F, s, sample_rows=ns)
    bits_whole = whole * R * C - 8.0 * meta(R)
    bits_part = part * ns * C - 8.0 * meta(ns)
    assert abs(bits_whole - bits_part * R / ns) <= 1e-9 * bits_whole
    if n >= R:
        assert whole == orc.estimate_bpp(w, S.BF16, F, s, sample_rows=R)


@pytest.mark.parametrize("iters", [0, 3, 12, 40])
def test_search_iters_bracket(orc, iters):
    w = S.lognormal_rows(96, 1024, seed=21)
    target = 3.0
    s = orc.search_scale(w, S.BF16, 8192, target, search_iters=iters)
    assert orc.estimate_bpp(w, S.BF16, 8192, s) <= target
    finer = 2.0 ** (np.log2(s) - 32.0 / 2.0 ** iters)
    assert orc.estimate_bpp(w, S.BF16, 8192, finer) > target
    # the compress call uses the same search
    st, blob, s2 = orc.compress(w, S.BF16, target, 8192, search_iters=iters)
    assert st == 0 and s2 == s


def test_compress_uses_the_sample_setting(orc):
    w = S.workload_weights(2, 600, 256)
    for n in (32, 256, 600):
        s = orc.search_scale(w, S.BF16, 4096, 3.0, sample_rows=n)
        st, blob, s2 = orc.compress(w, S.BF16, 3.0, 4096, sample_rows=n, rate_check=0)
        assert st == 0 and s2 == s
        # with the whole-tensor check: the searched scale, or a coarser one that meets the target
        st, blob, s3 = orc.compress(w, S.BF16, 3.0, 4096, sample_rows=n)
        assert st == 0 and s3 == orc.check_scale(w, S.BF16, 4096, 3.0, s) and s3 >= s
    st, _, _ = orc.compress(w, S.BF16, 3.0, 4096, sample_rows=0)
    assert st == orc.ERR_ARG


# ------------------------------------------------------------------------------------------
# The whole-tensor check of the searched scale
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("R,C,target", [(1024, 4096, 6.0), (2048, 2048, 6.0), (600, 2048, 4.5)])
def test_rate_check_on_heavy_tails(orc, R, C, target):
    """5b's recipe (int8 absmax of Laplace values) at reduced shapes: the 256-row sample misses
    rare values, its estimate undershoots the tensor's, and the check raises the scale until the
    whole-tensor estimate meets the target -- to the bisection's resolution (ten halvings of a
    step of at least 1/8 in log2 s, so within about 2^-13 of a doubling, a few thousandths of a
    bit per element) -- and the stored rate lands within 3% below it."""
    _, _, q = S.laplace_pair(R, C, seed=5)
    ss = orc.row_sumsq(q, S.INT8)
    s0 = orc.search_scale(q, S.INT8, 16384, target, sumsq=ss)
    full0 = orc.estimate_bpp(q, S.INT8, 16384, s0, sumsq=ss, sample_rows=R)
    assert full0 > target                            # the sample alone overshoots here
    s = orc.check_scale(q, S.INT8, 16384, target, s0, sumsq=ss)
    full = orc.estimate_bpp(q, S.INT8, 16384, s, sumsq=ss, sample_rows=R)
    assert s > s0
    assert target - 0.01 <= full <= target
    st, blob, s_c = orc.compress(q, S.INT8, target, 16384)
    assert st == 0 and s_c == s
    bpp = 8.0 * blob.size / q.size
    assert 0.97 * target <= bpp <= target


def test_rate_check_keeps_a_scale_that_already_meets_the_target(orc):
    """With every row sampled the sampled estimate is the whole tensor's: the check changes
    nothing; likewise on a light-tailed tensor whose sample already reaches the target."""
    w = S.lognormal_rows(96, 1024, seed=21)
    s0 = orc.search_scale(w, S.BF16, 8192, 3.0)
    assert orc.check_scale(w, S.BF16, 8192, 3.0, s0) == s0
    w = S.workload_weights(2, 1024, 1024)
    s0 = orc.search_scale(w, S.BF16, 8192, 4.0)
    if orc.estimate_bpp(w, S.BF16, 8192, s0, sample_rows=1024) <= 4.0:
        assert orc.check_scale(w, S.BF16, 8192, 4.0, s0) == s0
