"""The allocation-free decode (ep_decompress_noalloc) against ep_decompress with a prepared table
buffer: the same output bytes and error word, call after call on one GPU, the second call on a
smaller blob (the library's per-GPU scratch keeps the previous call's tables, which every call
rewrites whole)."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, ep_mod, host, log

pytestmark = pytest.mark.gpu


def _decode_both(gb):
    import torch

    ep = ep_mod()
    err_ref, ref = gb.decode()
    d_out = torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_noalloc(gb.d_blob, gb.info, d_out, d_err)
    assert st == 0, st
    torch.cuda.synchronize()
    npdt = {1: np.uint16, 2: np.uint16, 3: np.uint8, 4: np.int8, 5: np.uint32}[gb.info.dtype]
    got = host(d_out).view(npdt).reshape(gb.info.rows, gb.pitch())[:, :gb.info.cols]
    return err_ref, ref, int(host(d_err)[0]), got


@pytest.mark.parametrize("order", ["large-then-small", "wide-then-narrow"])
def test_noalloc_decode_matches_the_table_buffer_decode(orc, order):
    if order == "large-then-small":
        cases = [(2, 512, 1024, 64), (1, 256, 256, 64)]
    else:
        cases = [(3, 256, 1024, 128), ("5a", 32, 2048, 64)]
    for key, R, C, lanes in cases:
        log("noalloc", order, key, R, C, lanes)
        wl = S.WORKLOADS[key]
        w = S.workload_weights(key, R, C)
        st, blob, _ = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"],
                                   lanes=lanes)
        assert st == 0
        err_ref, ref, err, got = _decode_both(GpuBlob(blob))
        assert err_ref == 0 and err == 0
        assert np.array_equal(got, ref)
        st, oref, _, _ = orc.decompress(blob)
        assert st == 0 and np.array_equal(got, oref)


def test_noalloc_reports_a_corrupt_tile(orc):
    w = S.workload_weights(2, 256, 1024)
    st, blob, _ = orc.compress(w, S.BF16, 4.0, 8192)
    bad = blob.copy()
    bad[-64] ^= 0x5A
    err_ref, _, err, _ = _decode_both(GpuBlob(bad))
    assert err_ref & (1 << 7) and err == err_ref
