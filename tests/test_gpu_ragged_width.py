"""GPU parity for widths that are not a multiple of 8 (rows zero-padded to whole 8-vectors):
row sums, quantiser + histogram, LS terms, the fused decode (real columns compared; the padding
columns are the decoder's own) and the library's compress, against the oracle bit for bit."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, gpu_compress, gpu_quantize, gpu_row_lsq, gpu_row_sumsq, log

pytestmark = pytest.mark.gpu


def weights(dt, R, C, seed):
    if dt == S.FP8:
        return S.laplace_pair(R, C, seed=seed)[1]
    if dt == S.INT8:
        return S.laplace_pair(R, C, seed=seed)[2]
    if dt == S.FP16:
        return S.student_t_outliers(R, C, seed=seed)
    return S.lognormal_rows(R, C, seed=seed, dtype=dt)


DTS = [S.BF16, S.FP16, S.FP8, S.INT8, S.FP32]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("C", [1, 5, 13, 1001])
def test_ragged_width_encoder_kernels(orc, dt, C):
    log("ragged encoder kernels", dt, C)
    R = 70
    w = weights(dt, R, C, seed=60 + C)
    ss = gpu_row_sumsq(w, dt)
    ss_o = orc.row_sumsq(w, dt)
    assert np.array_equal(ss.view(np.uint64), ss_o.view(np.uint64))
    g = orc.gains(ss_o, C, 0.3)
    err, cos, fld, hist = gpu_quantize(w, dt, g)
    st, cos_o, fld_o = orc.quantize(w, dt, g)
    assert err == 0 and st == 0
    assert np.array_equal(cos, cos_o) and np.array_equal(fld, fld_o)
    assert np.array_equal(hist.astype(np.uint64), orc.histogram(cos_o, fld_o))
    num, den4 = gpu_row_lsq(w, dt, cos_o, fld_o)
    num_o, den4_o = orc.row_lsq(w, dt, cos_o, fld_o)
    assert np.array_equal(num.view(np.uint64), num_o.view(np.uint64))
    assert np.array_equal(den4, den4_o)


@pytest.mark.parametrize("dt,R,C,F", [(S.BF16, 300, 1001, 4096), (S.FP16, 64, 4099, 8192),
                                      (S.FP8, 37, 3333, 16384), (S.INT8, 128, 77, 4096),
                                      (S.FP32, 9, 5, 4096)], ids=str)
def test_ragged_width_decode_and_compress(orc, dt, R, C, F):
    log("ragged decode", dt, R, C)
    w = weights(dt, R, C, seed=61)
    st, blob_o, s_o = orc.compress(w, dt, 3.0, F)
    assert st == 0
    err, out = GpuBlob(blob_o).decode()
    st, ref, _, _ = orc.decompress(blob_o)
    assert err == 0 and out.shape == (R, C) and np.array_equal(out, ref)
    blob, s = gpu_compress(w, dt, 3.0, F)
    assert s == s_o and np.array_equal(blob, blob_o)


def test_ragged_width_high_level():
    import torch

    import entropy_coded_weight_ep_amd as ep

    log("ragged high level")
    w = S.lognormal_rows(300, 1001, seed=62)
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    c = ep.compress(t, ep.LatticeRANSConfig(target_bpp=3.0, tile_fields=4096, refine=3))
    r = ep.decompress(c)
    assert r.shape == t.shape and r.dtype == t.dtype
    rel = ((r.float() - t.float()).norm() / t.float().norm()).item()
    assert 0.0 < rel < 0.3
