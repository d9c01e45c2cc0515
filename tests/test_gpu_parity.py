"""GPU parity: every HIP kernel of libep.so against the CPU oracle, element by element, on seeded
synthetic inputs (integer and byte results bit-exact; the fp64 row sums and the decoded
containers are bit-exact as well, since both sides use the same rounded operations in the same
order).

Sizes span several tiles and ragged tails; the full-size workloads are in
test_gpu_fullsize.py.  Inputs come from ep_synth; expected values only from the oracle.
"""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import (GpuBlob, ep_mod, gpu_compress, gpu_quantize, gpu_row_lsq, gpu_row_sumsq,
                      log)

pytestmark = pytest.mark.gpu

DTYPES = [S.BF16, S.FP16, S.FP8, S.INT8]


def weights(dtype, R, C, seed):
    if dtype == S.FP16:
        return S.student_t_outliers(R, C, seed=seed)
    if dtype == S.FP8:
        return S.laplace_pair(R, C, seed=seed)[1]
    if dtype == S.INT8:
        return S.laplace_pair(R, C, seed=seed)[2]
    return S.lognormal_rows(R, C, seed=seed)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(64, 64), (130, 200), (7, 1032)])
def test_row_sumsq(orc, dtype, shape):
    log("row_sumsq", dtype, shape)
    w = weights(dtype, *shape, seed=11)
    got = gpu_row_sumsq(w, dtype)
    ref = orc.row_sumsq(w, dtype)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


@pytest.mark.parametrize("dtype", [S.FP8, S.INT8])
@pytest.mark.parametrize("cols", [131072, 131080, 28672 + 5])
def test_row_sumsq_wide_extremes(orc, dtype, cols):
    """fp8 and int8 rows are summed by one workgroup per row in any order (every partial sum
    is exact in fp64 up to 2^17 fp8 elements; wider fp8 rows take the left-to-right kernel).
    Rows of extreme magnitudes at and past that width, and a ragged one: the largest value, the
    smallest subnormal and zeros interleaved, alternating signs, and random codes, must give the
    oracle's sums bit for bit."""
    log("row_sumsq wide", dtype, cols)
    g = np.random.Generator(np.random.PCG64(29))
    big = 448.0 if dtype == S.FP8 else -128.0
    tiny = 2.0 ** -9 if dtype == S.FP8 else 1.0
    rows = [np.tile(np.array([big, tiny, 0.0, -big], np.float32), cols // 4 + 1)[:cols],
            np.full(cols, big, np.float32),
            np.where(np.arange(cols) % 2 == 0, tiny, -tiny).astype(np.float32),
            g.laplace(0.0, 30.0 if dtype == S.FP8 else 40.0, cols).astype(np.float32)]
    x = np.stack(rows)
    if dtype == S.INT8:
        x = np.clip(np.rint(x), -128, 127)
    else:
        x = np.clip(x, -448.0, 448.0)                 # finite codes only
    w = S.cast_container(x, dtype)
    got = gpu_row_sumsq(w, dtype)
    ref = orc.row_sumsq(w, dtype)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("s", [0.03, 0.4, 2.5])
def test_quantize_and_histogram(orc, dtype, s):
    log("quantize", dtype, s)
    w = weights(dtype, 96, 264, seed=5)
    ss = orc.row_sumsq(w, dtype)
    g = orc.gains(ss, w.shape[1], s)
    err, cos, fld, hist = gpu_quantize(w, dtype, g)
    st, cos_o, fld_o = orc.quantize(w, dtype, g)
    assert (err != 0) == (st != 0)
    if st == 0:
        assert np.array_equal(cos, cos_o)
        assert np.array_equal(fld, fld_o)
        assert np.array_equal(hist.astype(np.uint64), orc.histogram(cos_o, fld_o))
    else:
        assert err & (1 << 5)


def test_quantize_row_selection(orc):
    log("quantize row selection")
    w = S.lognormal_rows(300, 512, seed=3)
    ss = orc.row_sumsq(w, S.BF16)
    sel = np.array([(i * 300) // 256 for i in range(256)], np.int64)
    g = np.zeros(300, np.float32)
    g[sel] = orc.gains(ss[sel], 512, 0.3)
    err, cos, fld, hist = gpu_quantize(w, S.BF16, g, row_sel=sel)
    st, cos_o, fld_o = orc.quantize(w, S.BF16, g, row_sel=sel)
    assert err == 0 and st == 0
    assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)
    assert np.array_equal(hist.astype(np.uint64), orc.histogram(cos_o, fld_o))


def test_quantize_range_error(orc):
    log("quantize range")
    w = S.iid_normal(8, 64, seed=2)
    ss = orc.row_sumsq(w, S.BF16)
    g = orc.gains(ss, 64, 1e-6)
    err, *_ = gpu_quantize(w, S.BF16, g)
    assert err & (1 << 5)
    assert orc.quantize(w, S.BF16, g)[0] == orc.ERR_RANGE


def test_quantize_range_boundary(orc):
    """The range test |x| <= 65536 at its boundary and on non-finite inputs, one vector per call
    (the oracle stops at the first vector out of range): the GPU must flag exactly the vectors the
    oracle rejects and give the oracle's fields for the others.  bf16 holds 65536 and its upper
    neighbour 65792; fp32 holds 65536's neighbours one ulp away on both sides."""
    log("quantize range boundary")
    f32 = lambda b: float(np.array([b], np.uint32).view(np.float32)[0])
    # the field range |z| <= 32767 rejects |x| = 65536 already; values near 32767 probe that
    # second boundary (32640 is bf16's largest value below it)
    specials = [65536.0, 65792.0, f32(0x47800001), f32(0x477FFFFF), np.inf, np.nan,
                f32(0x7F7FFFFF), f32(0x00000001), 0.0, 1e30,
                32640.0, 32766.5, 32767.0, 32767.5, 32768.0]
    rng = np.random.Generator(np.random.PCG64(11))
    n_ok = n_bad = 0
    for dt in (S.BF16, S.FP32):
        for v in specials:
            for sign in (1.0, -1.0):
                x = rng.normal(0.0, 3.0, 8).astype(np.float32)
                x[int(rng.integers(8))] = np.float32(sign * v)
                w = S.cast_container(x.reshape(1, 8), dt)
                g = np.ones(1, np.float32)
                err, cos, fld, _ = gpu_quantize(w, dt, g, with_hist=False)
                st, cos_o, fld_o = orc.quantize(w, dt, g)
                assert (err != 0) == (st != 0), (dt, sign * v, err, st)
                if st == 0:
                    n_ok += 1
                    assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)
                else:
                    n_bad += 1
                    assert st == orc.ERR_RANGE and err == 1 << 5
                    assert cos[0] == 0 and not fld.any()   # flagged vectors are written as 0
    assert n_ok >= 12 and n_bad >= 24


def test_quantize_odd_parity_fixups(orc):
    """Vectors whose rounded sum is odd for both candidates, with ties in the worst residual
    (several coordinates at the same distance from their integers, either sign) and zero
    residuals: the fix-up must move the same coordinate in the same direction as the oracle."""
    log("quantize parity fix-ups")
    rng = np.random.Generator(np.random.PCG64(12))
    rows = []
    for _ in range(2048):
        base = rng.integers(-6, 7, 8).astype(np.float32)
        frac = rng.choice(np.array([0.0, 0.25, -0.25, 0.375, -0.375, 0.125, 0.5, -0.5],
                                   np.float32), 8)
        rows.append(base + frac)
    x = np.stack(rows).astype(np.float32)
    for dt in (S.BF16, S.FP32):
        w = S.cast_container(x, dt)
        g = np.ones(len(rows), np.float32)
        err, cos, fld, _ = gpu_quantize(w, dt, g, with_hist=False)
        st, cos_o, fld_o = orc.quantize(w, dt, g)
        assert err == 0 and st == 0
        assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)


def test_quantize_special_vectors(orc):
    """Hand-worked E8 cases (tests/golden/e8_cases.txt) through the GPU quantiser with unit gain:
    cases that bf16 holds exactly must give the worked answer; all must match the oracle."""
    from test_oracle_e8 import golden_cases

    log("quantize golden")
    cases = golden_cases()
    x = np.stack([c[0] for c in cases]).astype(np.float32)
    bits = S.cast_container(x, S.BF16)
    exact = np.all(S.container_to_float(bits, S.BF16) == x, axis=1)
    w = np.ascontiguousarray(bits.reshape(len(cases), 8))
    g = np.ones(len(cases), np.float32)
    err, cos, fld, _ = gpu_quantize(w, S.BF16, g)
    st, cos_o, fld_o = orc.quantize(w, S.BF16, g)
    assert err == 0 and st == 0
    assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)
    assert exact.sum() >= 5
    for i, c in enumerate(cases):
        if exact[i]:
            assert cos[i] == c[1], c[4]
            assert np.array_equal(fld[8 * i:8 * i + 8], c[3]), c[4]


@pytest.mark.parametrize("dtype", DTYPES)
def test_row_lsq(orc, dtype):
    log("row_lsq", dtype)
    w = weights(dtype, 70, 392, seed=8)
    ss = orc.row_sumsq(w, dtype)
    g = orc.gains(ss, 392, 0.5)
    st, cos, fld = orc.quantize(w, dtype, g)
    assert st == 0
    num, den4 = gpu_row_lsq(w, dtype, cos, fld)
    num_o, den4_o = orc.row_lsq(w, dtype, cos, fld)
    assert np.array_equal(num.view(np.uint64), num_o.view(np.uint64))
    assert np.array_equal(den4, den4_o)


# (key, rows, cols) -- reduced shapes of the five workloads, several tiles each; the ragged
# cases leave a partial last tile.
DECODE_CASES = [
    (1, 256, 256),          # 16 tiles of 512 vectors, J = 8
    (2, 512, 1024),         # J = 16
    (2, 200, 776),          # ragged: 19400 vectors, last tile 968 of 1024
    (3, 256, 1024),         # fp16, heavy tails: wide-alphabet path
    (4, 96, 3072),          # J = 16, tiles span rows
    ("5a", 64, 2048),       # fp8, J = 32
    ("5b", 64, 2048),       # int8, J = 32, wide alphabet
    ("5b", 37, 1000),       # ragged J = 32, 3 tiles
    (1, 3, 8),              # one vector per row, single ragged tile
]


def _oracle_blob(orc, key, R, C, target=None):
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    st, blob, s = orc.compress(w, wl["dtype"], target or wl["target_bpp"], wl["tile_fields"])
    assert st == 0
    return w, blob


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_decode_matches_oracle(orc, case):
    key, R, C = case
    log("decode", case)
    w, blob = _oracle_blob(orc, key, R, C)
    gb = GpuBlob(blob)
    err, out = gb.decode()
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0 and err == 0
    assert out.shape == ref.shape and out.dtype == ref.dtype
    assert np.array_equal(out, ref)
    # determinism: a second launch gives the same bytes
    err2, out2 = gb.decode()
    assert err2 == 0 and np.array_equal(out2, out)


@pytest.mark.parametrize("target", [0.001, 1.0, 8.0, 11.0])
def test_decode_extreme_rates(orc, target):
    log("decode rate", target)
    w, blob = _oracle_blob(orc, 2, 128, 1024, target=target)
    err, out = GpuBlob(blob).decode()
    st, ref, _, _ = orc.decompress(blob)
    assert err == 0 and np.array_equal(out, ref)


def test_decode_zero_matrix(orc):
    log("decode zeros")
    z = np.zeros((64, 512), np.uint16)
    st, blob, s = orc.compress(z, S.BF16, 3.0, 4096)
    err, out = GpuBlob(blob).decode()
    assert err == 0 and np.all(out == 0)


def test_decode_detects_corrupt_tile(orc):
    log("decode corrupt")
    w, blob = _oracle_blob(orc, 2, 256, 1024)
    info = orc.blob_fields(blob)
    bad = blob.copy()
    bad[-64] ^= 0x5A                                  # a payload word of the last tile
    gb = GpuBlob(bad)
    err, _ = gb.decode()
    assert err & (1 << 7)
    assert orc.decompress(bad)[0] == orc.ERR_CORRUPT
    assert info["tiles"] > 1


LAYOUT_CASES = [
    (2, 512, 1024, None),       # J = 16
    (2, 200, 776, None),        # ragged
    (3, 256, 1024, None),       # wide alphabet
    ("5a", 64, 2048, None),     # J = 32
    ("5b", 64, 2048, None),     # J = 32, wide alphabet, 6.6 bpp
    ("5b", 37, 1000, None),     # ragged J = 32
    (2, 128, 1024, 11.0),       # the highest rate: phases consume more than a small ring holds
    (1, 256, 256, 8.0),         # J = 8
]


@pytest.mark.parametrize("flags", ["LINEAR", "RING", "RING_MIN"])
@pytest.mark.parametrize("case", LAYOUT_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-{c[3]}")
def test_decode_word_layouts_match_oracle(orc, case, flags):
    """Each tile's words held whole in LDS, or streamed through a ring (automatic size, and the
    smallest ring, which refills in the middle of phases): the same bytes as the oracle."""
    key, R, C, target = case
    log("decode layout", case, flags)
    ep = ep_mod()
    w, blob = _oracle_blob(orc, key, R, C, target=target)
    gb = GpuBlob(blob)
    err, out = gb.decode(flags=getattr(ep, "EP_DECODE_" + flags))
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0 and err == 0
    assert np.array_equal(out, ref)


def test_decode_ring_detects_corrupt_tile(orc):
    log("decode ring corrupt")
    ep = ep_mod()
    w, blob = _oracle_blob(orc, 2, 256, 1024)
    bad = blob.copy()
    bad[-64] ^= 0x5A                                  # a payload word of the last tile
    gb = GpuBlob(bad)
    for flags in (ep.EP_DECODE_RING, ep.EP_DECODE_RING_MIN):
        err, _ = gb.decode(flags=flags)
        assert err & (1 << 7)


def test_decode_batch_matches_oracle(orc):
    """One batched decode of 40 blobs (two launches of up to 32; some ragged, some with wide
    alphabets, different shapes) writes what 40 oracle decodes write."""
    import torch

    ep = ep_mod()
    blobs, refs = [], []
    shapes = [(64, 3072), (40, 1000), (96, 512), (8, 8), (128, 1024)]
    for i in range(40):
        R, C = shapes[i % len(shapes)]
        key = 4 if i % 3 else 2
        w = S.workload_weights(key, R, C, i)
        target = 3.0 if i % 4 else 7.0                # 7 bpp: wide alphabets
        st, blob, s = orc.compress(w, S.BF16, target, 8192)
        assert st == 0
        st, ref, _, _ = orc.decompress(blob)
        assert st == 0
        blobs.append(GpuBlob(blob))
        refs.append(ref)
    log("decode batch", len(blobs))
    outs = [torch.zeros(b.out_bytes(), dtype=torch.uint8, device="cuda") for b in blobs]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_batch([b.d_blob for b in blobs], [b.info for b in blobs],
                                [b.d_tab for b in blobs], outs, d_err)
    assert st == 0
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0
    for b, o, ref in zip(blobs, outs, refs):
        got = o.cpu().numpy().view(np.uint16).reshape(b.info.rows, b.info.cols)
        assert np.array_equal(got, ref)


def test_decode_fp8_batch_mixed_bounds(orc):
    """A batch of fp8 blobs at 16384-field tiles where some blobs are bounded (values within
    +-448) and some are not: the whole batch takes the clamped conversion, and a batch of
    bounded blobs alone the unclamped one; both must write what the oracle writes."""
    import torch

    ep = ep_mod()
    wl = S.WORKLOADS["5a"]
    blobs, refs = [], []
    for i in range(6):
        w = S.workload_weights("5a", 16, 4096, i)
        st, blob, s = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
        assert st == 0
        if i % 3 == 2:                                  # one row scale far past the bound
            st, info = ep.ep_blob_parse(blob)
            assert st == 0
            blob = blob.copy()
            blob[info.off_alpha:info.off_alpha + 4] = np.array([500.0], np.float32).view(np.uint8)
        st, ref, _, _ = orc.decompress(blob)
        assert st == 0
        blobs.append(GpuBlob(blob))
        refs.append(ref)
    assert sorted({b.info.bounded for b in blobs}) == [0, 1]
    log("decode fp8 batch, mixed bounds")
    for sel in (range(6), [i for i in range(6) if blobs[i].info.bounded]):
        bs = [blobs[i] for i in sel]
        outs = [torch.zeros(b.out_bytes(), dtype=torch.uint8, device="cuda") for b in bs]
        d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
        st = ep.ep_decompress_batch([b.d_blob for b in bs], [b.info for b in bs],
                                    [b.d_tab for b in bs], outs, d_err)
        assert st == 0
        torch.cuda.synchronize()
        assert int(d_err.item()) == 0
        for i, o in zip(sel, outs):
            got = o.cpu().numpy().reshape(blobs[i].info.rows, blobs[i].info.cols)
            assert np.array_equal(got, refs[i].view(np.uint8))


def test_decode_batch_rejects_mixed_containers(orc):
    import torch

    ep = ep_mod()
    a = GpuBlob(_oracle_blob(orc, 2, 64, 1024)[1])
    w = S.workload_weights(3, 64, 1024)
    st, blob, s = orc.compress(w, S.FP16, 3.0, 8192)
    b = GpuBlob(blob)
    outs = [torch.zeros(x.out_bytes(), dtype=torch.uint8, device="cuda") for x in (a, b)]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert ep.ep_decompress_batch([a.d_blob, b.d_blob], [a.info, b.info], [a.d_tab, b.d_tab],
                                  outs, d_err) == ep.EP_ERR_ARG


def test_decode_layout_flags_rejected(orc):
    import torch

    ep = ep_mod()
    w, blob = _oracle_blob(orc, 1, 256, 256)
    gb = GpuBlob(blob)
    d_out = torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for flags in (8, ep.EP_DECODE_LINEAR | ep.EP_DECODE_RING, 3 | 4):
        assert ep.ep_decompress_ex(gb.d_blob, gb.info, gb.d_tab, d_out, d_err, flags) == \
            ep.EP_ERR_ARG
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0


@pytest.mark.parametrize("case", [(1, 256, 256), (2, 256, 1024), (3, 128, 1024),
                                  ("5a", 32, 2048), ("5b", 32, 2048), (2, 200, 776)],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_compress_blob_matches_oracle(orc, case):
    """The library's compress (GPU quantiser, histogram, row sums and LS terms; host tables,
    encoder and search) writes the oracle's blob byte for byte."""
    key, R, C = case
    log("compress", case)
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    blob, s = gpu_compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
    st, blob_o, s_o = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
    assert st == 0
    assert s == s_o
    assert blob.size == blob_o.size and np.array_equal(blob, blob_o)


def test_high_level_roundtrip(orc):
    """The usage of the design page: compress at 3.5 bpp, decompress, same shape and dtype."""
    import torch

    import entropy_coded_weight_ep_amd as ep

    log("high level")
    w = S.workload_weights(1)
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    cfg = ep.LatticeRANSConfig(target_bpp=3.5, tile_fields=4096)
    c = ep.compress(t, cfg)
    r = ep.decompress(c, cfg)
    assert r.shape == t.shape and r.dtype == t.dtype
    rel = ((r.float() - t.float()).norm() / t.float().norm()).item()
    assert 0.0 < rel < 0.3
    assert abs(c.actual_bpp - 8.0 * c.blob.size / w.size) < 1e-12
    st, blob_o, _ = orc.compress(w, S.BF16, 3.5, 4096)
    assert np.array_equal(c.blob, blob_o)


def _midpoint_alphas(n, seed):
    """fp32 row scales a for which fp16(fp32(a * p)) differs from a single rounding of the exact
    product a * p for some half-integer p in [-32, 32]: the products land on fp16 midpoints only
    after the fp32 rounding.  The decoder must round twice (fp32, then the container)."""
    g = np.random.Generator(np.random.PCG64(seed))
    p = np.arange(-64, 65, dtype=np.float64) / 2
    out = []
    while len(out) < n:
        a = np.float32(g.uniform(0.004, 0.06))
        y32 = (a * p.astype(np.float32)).astype(np.float32)
        if np.any(y32.astype(np.float16) != (float(a) * p).astype(np.float16)):
            out.append(a)
    return np.array(out, np.float32)


def test_decode_double_rounding_midpoints(orc):
    """Row scales chosen so that many fp32 products sit on fp16 rounding midpoints."""
    log("decode midpoints")
    w, blob = _oracle_blob(orc, 3, 64, 1024)
    info = orc.blob_fields(blob)
    o = 64 + info["table_bytes"]
    bad = blob.copy()
    alphas = _midpoint_alphas(64, seed=17)
    bad[o:o + 4 * 64] = alphas.view(np.uint8)
    st, ref, cos, fld = orc.decompress(bad, want_fields=True)
    assert st == 0
    # how many elements would a single rounding get wrong?
    z = fld.reshape(-1, 8).astype(np.int64)
    z[:, 7] = 2 * z[:, 7] + (z[:, :7].sum(axis=1) & 1)
    p = (z + 0.5 * cos[:, None]).reshape(64, 1024)
    y32 = (alphas[:, None] * p.astype(np.float32)).astype(np.float32)
    single = (alphas[:, None].astype(np.float64) * p).astype(np.float16)
    n_mid = int(np.sum(y32.astype(np.float16) != single))
    assert n_mid > 10
    err, out = GpuBlob(bad).decode()
    assert err == 0
    assert np.array_equal(out, ref), f"{int(np.sum(out != ref))} elements differ"


@pytest.mark.parametrize("key,shape", [(2, (64, 1024)), (3, (64, 1024)), ("5a", (32, 2048)),
                                       ("5b", (32, 2048))], ids=lambda c: str(c))
def test_decode_container_edges(orc, key, shape):
    """Row scales swept over 1e-40 .. 1e4 with both signs, so that the decoded products reach
    container subnormals, saturation (fp8 at +-448, int8 at -128 / 127) and overflow (fp16 to
    +-inf); the GPU conversions must match the oracle's bit for bit."""
    R, C = shape
    log("decode edges", key)
    w, blob = _oracle_blob(orc, key, R, C)
    info = orc.blob_fields(blob)
    o = 64 + info["table_bytes"]
    g = np.random.Generator(np.random.PCG64(23))
    alphas = (10.0 ** np.linspace(-40, 4, R) * np.where(g.random(R) < 0.5, -1.0, 1.0))
    alphas = alphas.astype(np.float32)
    bad = blob.copy()
    bad[o:o + 4 * R] = alphas.view(np.uint8)
    st, ref, _, _ = orc.decompress(bad)
    assert st == 0
    err, out = GpuBlob(bad).decode()
    assert err == 0
    assert np.array_equal(out, ref), f"{int(np.sum(out != ref))} elements differ"


@pytest.mark.parametrize("shape", [(32, 2048), (64, 28672)], ids=lambda c: f"{c[0]}x{c[1]}")
def test_fp8_bounded_and_clamped_decodes(orc, shape):
    """An fp8 blob whose decoded values provably stay within +-448 (`bounded`) is converted
    without the saturation clamp; raising one row scale past the bound sends the same blob
    through the clamped conversion.  Both must equal the oracle's decode bit for bit, at a
    16384-field tile shape (32 vectors per lane, the two-workgroups-per-CU ring launch)."""
    import entropy_coded_weight_ep_amd as ep

    R, C = shape
    log("fp8 bounded / clamped", shape)
    wl = S.WORKLOADS["5a"]
    w = S.workload_weights("5a", R, C)
    st, blob, s = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
    assert st == 0
    st, info = ep.ep_blob_parse(blob)
    assert st == 0 and info.bounded == 1
    bad = blob.copy()
    for r in range(0, R, 7):                        # a few rows far past the bound
        bad[info.off_alpha + 4 * r:info.off_alpha + 4 * r + 4] = \
            np.array([(-1.0) ** r * 300.0], np.float32).view(np.uint8)
    st, info_bad = ep.ep_blob_parse(bad)
    assert st == 0 and info_bad.bounded == 0
    for b in (blob, bad):
        st, ref, _, _ = orc.decompress(b)
        assert st == 0
        err, out = GpuBlob(b).decode()
        assert err == 0
        assert np.array_equal(out, ref), f"{int(np.sum(out != ref))} elements differ"
    # the clamped blob really saturates somewhere
    assert np.any((ref.view(np.uint8) & 0x7F) == 0x7E)


def test_blob_with_nonfinite_scale_is_rejected(orc):
    import entropy_coded_weight_ep_amd as ep

    w, blob = _oracle_blob(orc, 1, 64, 256)
    info = orc.blob_fields(blob)
    o = 64 + info["table_bytes"]
    bad = blob.copy()
    bad[o:o + 4] = np.array([np.inf], np.float32).view(np.uint8)
    assert ep.ep_blob_parse(bad)[0] == ep.EP_ERR_CORRUPT


def test_fp8_every_code_in_encoder_kernels(orc):
    """Rows holding every fp8 e4m3fn code but the two NaNs, at scales from tiny to large, plus a
    row with a NaN: row sums, quantiser and LS terms against the oracle (the GPU widens fp8 with
    the hardware conversion, the oracle from the format's definition)."""
    log("fp8 every code")
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)   # 254 codes
    g = np.random.Generator(np.random.PCG64(77))
    rows = [g.permutation(codes) for _ in range(12)]
    w = np.stack([np.concatenate([r, r[:2]]) for r in rows])                  # 12 x 256
    ss = gpu_row_sumsq(w, S.FP8)
    ss_o = orc.row_sumsq(w, S.FP8)
    assert np.array_equal(ss.view(np.uint64), ss_o.view(np.uint64))
    for s in (0.05, 1.0, 30.0):
        gn = orc.gains(ss_o, 256, s)
        err, cos, fld, hist = gpu_quantize(w, S.FP8, gn)
        st, cos_o, fld_o = orc.quantize(w, S.FP8, gn)
        assert (err != 0) == (st != 0)
        if st == 0:
            assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)
            num, den4 = gpu_row_lsq(w, S.FP8, cos_o, fld_o)
            num_o, den4_o = orc.row_lsq(w, S.FP8, cos_o, fld_o)
            assert np.array_equal(num.view(np.uint64), num_o.view(np.uint64))
            assert np.array_equal(den4, den4_o)
    bad = w.copy()
    bad[3, 100] = 0x7F                                                         # NaN
    ss = gpu_row_sumsq(bad, S.FP8)
    assert np.isnan(ss[3]) and np.isnan(orc.row_sumsq(bad, S.FP8)[3])
    assert np.array_equal(np.delete(ss, 3).view(np.uint64), np.delete(ss_o, 3).view(np.uint64))


def test_compress_rejects_undecodable_tile_sizes():
    import torch

    import entropy_coded_weight_ep_amd as ep

    log("compress tile sizes")
    t = torch.from_numpy(S.iid_normal(64, 256, seed=3).view(np.int16)).view(torch.bfloat16).cuda()
    for F in (512, 2048, 12288, 32768):
        with pytest.raises(ep.EPError):
            ep.compress(t, ep.LatticeRANSConfig(target_bpp=3.0, tile_fields=F))
    c = ep.compress(t, ep.LatticeRANSConfig(target_bpp=3.0, tile_fields=16384))
    assert ep.decompress(c).shape == t.shape


# Rows of at least 64 * 32 vectors with wide alphabets at 16384-field tiles: the decoder keeps
# two row scales per wave (a tile then spans at most two rows) and runs 12-wave workgroups.
LONG_ROWS = [
    ("5b", 16, 28672, 6.0),      # int8, tiles crossing rows
    ("5b", 7, 16400, 6.0),       # 2050 vectors per row, ragged last tile
    (3, 9, 16384, 7.0),          # fp16, exactly 2048 vectors per row
    (2, 5, 20000, 8.0),          # bf16
]


@pytest.mark.parametrize("case", LONG_ROWS)
def test_decode_long_rows_wide_alphabet(orc, case):
    key, R, C, target = case
    ep = ep_mod()
    log("decode long rows", case)
    w = S.workload_weights(key, R, C)
    dt = S.WORKLOADS[key]["dtype"]
    st, blob, _ = orc.compress(w, dt, target, 16384)
    assert st == 0
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0
    gb = GpuBlob(blob)
    assert gb.info.big_alphabet and (C + 7) // 8 >= 2048
    for flags in (None, ep.EP_DECODE_LINEAR, ep.EP_DECODE_RING, ep.EP_DECODE_RING_MIN):
        err, out = gb.decode(flags=flags)
        assert err == 0 and np.array_equal(out, ref), flags


def test_decode_batch_long_rows(orc):
    """Two long-row wide-alphabet blobs in one batched call (the two-row path), and the same two
    with a short-row blob added (the per-vector scales): all as the oracle writes them."""
    import torch

    ep = ep_mod()
    log("decode batch long rows")
    cases = [("5b", 16, 28672, 6.0, 0), ("5b", 7, 16400, 6.0, 1), ("5b", 24, 2048, 6.0, 2)]
    blobs, refs = [], []
    for key, R, C, target, i in cases:
        w = S.workload_weights(key, R, C, i)
        st, blob, _ = orc.compress(w, S.WORKLOADS[key]["dtype"], target, 16384)
        assert st == 0
        st, ref, _, _ = orc.decompress(blob)
        assert st == 0
        blobs.append(GpuBlob(blob))
        refs.append(ref)
    for sel in ([0, 1], [0, 1, 2]):
        outs = [torch.zeros(blobs[i].out_bytes(), dtype=torch.uint8, device="cuda") for i in sel]
        d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
        st = ep.ep_decompress_batch([blobs[i].d_blob for i in sel], [blobs[i].info for i in sel],
                                    [blobs[i].d_tab for i in sel], outs, d_err)
        assert st == 0
        torch.cuda.synchronize()
        assert int(d_err.item()) == 0
        for i, o in zip(sel, outs):
            b = blobs[i]
            got = o.cpu().numpy().view(np.int8).reshape(b.info.rows, b.pitch())[:, :b.info.cols]
            assert np.array_equal(got, refs[i])
