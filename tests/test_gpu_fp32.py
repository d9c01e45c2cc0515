"""GPU parity for the fp32 container: row sums, quantiser + histogram, LS terms, the fused
decode (fast and exact-half scaling paths, ragged tiles, every tile size, wide alphabets) and
the library's compress, each against the oracle bit for bit.  Inputs: seeded fp32 weights with
log-normal row scales and Student-t tails (ep_synth)."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, gpu_compress, gpu_quantize, gpu_row_lsq, gpu_row_sumsq, log

pytestmark = pytest.mark.gpu

FP32 = S.FP32


def weights(R, C, seed, heavy=False):
    if heavy:
        return S.student_t_outliers(R, C, seed=seed, dtype=FP32)
    return S.lognormal_rows(R, C, seed=seed, dtype=FP32)


@pytest.mark.parametrize("shape", [(64, 64), (130, 200), (7, 1032)])
def test_fp32_row_stats(orc, shape):
    log("fp32 row stats", shape)
    w = weights(*shape, seed=31)
    got = gpu_row_sumsq(w, FP32)
    assert np.array_equal(got.view(np.uint64), orc.row_sumsq(w, FP32).view(np.uint64))
    g = orc.gains(orc.row_sumsq(w, FP32), shape[1], 0.4)
    st, cos, fld = orc.quantize(w, FP32, g)
    assert st == 0
    num, den4 = gpu_row_lsq(w, FP32, cos, fld)
    num_o, den4_o = orc.row_lsq(w, FP32, cos, fld)
    assert np.array_equal(num.view(np.uint64), num_o.view(np.uint64))
    assert np.array_equal(den4, den4_o)


@pytest.mark.parametrize("s", [0.03, 0.4, 2.5])
def test_fp32_quantize_and_histogram(orc, s):
    log("fp32 quantize", s)
    w = weights(96, 264, seed=32, heavy=True)
    g = orc.gains(orc.row_sumsq(w, FP32), 264, s)
    err, cos, fld, hist = gpu_quantize(w, FP32, g)
    st, cos_o, fld_o = orc.quantize(w, FP32, g)
    assert err == 0 and st == 0
    assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)
    assert np.array_equal(hist.astype(np.uint64), orc.histogram(cos_o, fld_o))


# (rows, cols, target bpp, tile fields, heavy tails)
DECODE = [
    (256, 256, 3.5, 4096, False),      # J = 8
    (512, 1024, 4.0, 8192, False),     # J = 16
    (200, 776, 4.0, 8192, False),      # ragged last tile
    (64, 2048, 2.0, 16384, False),     # J = 32
    (37, 1000, 6.0, 16384, True),      # ragged J = 32, wide alphabet
    (256, 1024, 2.5, 8192, True),      # wide alphabet
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"{c[0]}x{c[1]}-{c[2]}-F{c[3]}")
def test_fp32_decode_matches_oracle(orc, case):
    R, C, target, F, heavy = case
    log("fp32 decode", case)
    w = weights(R, C, seed=33, heavy=heavy)
    st, blob, s = orc.compress(w, FP32, target, F)
    assert st == 0
    err, out = GpuBlob(blob).decode()
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0 and err == 0
    assert out.dtype == np.uint32 and np.array_equal(out, ref)


def test_fp32_decode_scale_edges(orc):
    """Row scales swept over 1e-40 .. 1e4 with both signs: products reach fp32 subnormals (the
    blob then needs the exact-half path) and large magnitudes."""
    log("fp32 edges")
    R, C = 64, 1024
    w = weights(R, C, seed=34)
    st, blob, s = orc.compress(w, FP32, 4.0, 8192)
    info = orc.blob_fields(blob)
    o = 64 + info["table_bytes"]
    g = np.random.Generator(np.random.PCG64(35))
    alphas = (10.0 ** np.linspace(-40, 4, R) * np.where(g.random(R) < 0.5, -1.0, 1.0))
    bad = blob.copy()
    bad[o:o + 4 * R] = alphas.astype(np.float32).view(np.uint8)
    st, ref, _, _ = orc.decompress(bad)
    assert st == 0
    gb = GpuBlob(bad)
    assert gb.info.tiny_scale == 1
    err, out = gb.decode()
    assert err == 0
    assert np.array_equal(out, ref), f"{int(np.sum(out != ref))} elements differ"


@pytest.mark.parametrize("case", [(256, 1024, 4.0, 8192), (200, 776, 3.0, 4096),
                                  (32, 2048, 1.5, 16384)], ids=str)
def test_fp32_compress_blob_matches_oracle(orc, case):
    R, C, target, F = case
    log("fp32 compress", case)
    w = weights(R, C, seed=36)
    blob, s = gpu_compress(w, FP32, target, F)
    st, blob_o, s_o = orc.compress(w, FP32, target, F)
    assert st == 0 and s == s_o
    assert blob.size == blob_o.size and np.array_equal(blob, blob_o)


def test_fp32_high_level_roundtrip():
    import torch

    import entropy_coded_weight_ep_amd as ep

    log("fp32 high level")
    w = weights(128, 512, seed=37)
    t = torch.from_numpy(w.view(np.float32)).cuda()
    c = ep.compress(t, ep.LatticeRANSConfig(target_bpp=3.0, tile_fields=4096))
    r = ep.decompress(c)
    assert r.dtype == torch.float32 and r.shape == t.shape
    rel = ((r - t).norm() / t.norm()).item()
    assert 0.0 < rel < 0.3
