"""GPU parity for escapes: tensors whose full histogram gives some field table more than 2^12
distinct values.  The library's compress (host table build with escapes, device exception list,
device tile encoder with substitutes) must write the oracle's blob byte for byte, and its decode
(tiles, then the patch of the escaped vectors) must write the oracle's decode exactly, in every
container, tile size and words layout, alone and in a batch.  Expected values come only from the
oracle; inputs from ep_synth.
"""
import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, dev, ep_mod, gpu_compress, host, log

pytestmark = pytest.mark.gpu


def _escape_weights(dt):
    if dt in (S.FP8, S.INT8):                       # few container codes: wide normal rows
        return S.iid_normal(512, 1024, seed=9, sigma=1.0 if dt == S.FP8 else 40.0, dtype=dt)
    return S.student_t_outliers(512, 1024, seed=11, nu=2.0, scale=0.02, dtype=dt)


CASES = [
    (S.FP16, 4096),
    (S.FP16, 8192),
    (S.FP16, 16384),
    (S.BF16, 8192),
    (S.FP32, 8192),
    (S.FP8, 8192),
    (S.INT8, 16384),
]


def _oracle(orc, w, dt, F, s):
    st, blob, _ = orc.compress(w, dt, 3.0, F, force_s=s)
    assert st == 0
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0
    return blob, ref


@pytest.mark.parametrize("dt,F", CASES)
def test_escape_compress_and_decode(orc, dt, F):
    ep = ep_mod()
    w = _escape_weights(dt)
    s = 1.0 / 1000.0
    log("escape", dt, F)
    blob_o, ref = _oracle(orc, w, dt, F, s)
    assert orc.blob_exceptions(blob_o) > 0
    blob, _ = gpu_compress(w, dt, 3.0, F, force_scale=s)
    assert np.array_equal(blob, blob_o)
    gb = GpuBlob(blob)
    assert gb.info.n_exceptions == orc.blob_exceptions(blob_o)
    for flags in (None, ep.EP_DECODE_LINEAR, ep.EP_DECODE_RING, ep.EP_DECODE_RING_MIN):
        err, out = gb.decode(flags=flags)
        assert err == 0 and np.array_equal(out, ref.view(out.dtype)), flags


def test_escape_nearly_every_vector(orc):
    """Normal rows at s = 1/3000: each field table keeps 4096 of its ~20000 values, and almost
    every vector is listed as an exception (the decoder rewrites nearly all of them)."""
    w = S.iid_normal(512, 1024, seed=9)
    s = 1.0 / 3000.0
    log("escape nearly all")
    blob_o, ref = _oracle(orc, w, S.BF16, 8192, s)
    assert orc.blob_exceptions(blob_o) > 60000
    blob, _ = gpu_compress(w, S.BF16, 3.0, 8192, force_scale=s)
    assert np.array_equal(blob, blob_o)
    err, out = GpuBlob(blob).decode()
    assert err == 0 and np.array_equal(out, ref)


def test_escape_batch(orc):
    """A batched decode of blobs with and without exception lists."""
    import torch

    ep = ep_mod()
    log("escape batch")
    blobs, refs = [], []
    for i in range(5):
        if i % 2 == 0:
            w = S.student_t_outliers(512, 1024, seed=11 + i, nu=2.0, scale=0.02, dtype=S.FP16)
            blob, ref = _oracle(orc, w, S.FP16, 8192, 1.0 / 1000.0)
            assert orc.blob_exceptions(blob) > 0
        else:
            w = S.student_t_outliers(96, 1000, seed=i, dtype=S.FP16)
            blob, ref = _oracle(orc, w, S.FP16, 8192, 0.0)
            assert orc.blob_exceptions(blob) == 0
        blobs.append(GpuBlob(blob))
        refs.append(ref)
    outs = [torch.zeros(b.out_bytes(), dtype=torch.uint8, device="cuda") for b in blobs]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_batch([b.d_blob for b in blobs], [b.info for b in blobs],
                                [b.d_tab for b in blobs], outs, d_err)
    assert st == 0
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0
    for b, o, ref in zip(blobs, outs, refs):
        got = host(o).view(np.uint16).reshape(b.info.rows, b.pitch())[:, : b.info.cols]
        assert np.array_equal(got, ref)


def test_escape_bad_entries(orc):
    """An exception count the blob cannot hold is rejected before any launch; an entry that names
    a vector past the end (a device copy that differs from the parsed one) is reported as a
    corrupt blob by the patch kernel's own bounds check and not written."""
    import torch

    ep = ep_mod()
    w = _escape_weights(S.FP16)
    blob, ref = _oracle(orc, w, S.FP16, 8192, 1.0 / 1000.0)
    gb = GpuBlob(blob)
    info = gb.info
    log("escape bad entries")
    d_out = torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    n0 = info.n_exceptions
    info.n_exceptions = info.rows * ((info.cols + 7) // 8) + 1
    assert ep.ep_decompress(gb.d_blob, info, gb.d_tab, d_out, d_err) == ep.EP_ERR_ARG
    info.n_exceptions = n0
    bad = blob.copy()
    o = info.off_exceptions
    bad[o: o + 4].view(np.uint32)[0] = 0x7FFFFFFF
    d_bad = dev(bad)
    assert ep.ep_decompress(d_bad, info, gb.d_tab, d_out, d_err) == 0
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) & (1 << ep.EP_ERR_CORRUPT)
    # the other entries are still patched: only the first vector's row can differ
    got = host(d_out).view(np.uint16).reshape(info.rows, gb.pitch())[:, : info.cols]
    v0 = int(blob[o: o + 4].view(np.uint32)[0]) & 0x7FFFFFFF
    r0 = v0 // ((info.cols + 7) // 8)
    keep = np.ones(info.rows, bool)
    keep[r0] = False
    assert np.array_equal(got[keep], ref.view(np.uint16)[keep])


@pytest.mark.parametrize("F", [4096, 16384])
def test_escape_ragged_width(orc, F):
    """Escapes in a tensor whose width is not a multiple of 8 (zero-padded last vector of each
    row) and whose last tile is partly filled: the patched vectors land in the padded rows the
    decoder writes, and the visible columns match the oracle."""
    w = S.iid_normal(509, 1001, seed=9)
    s = 1.0 / 1000.0
    log("escape ragged", F)
    blob_o, ref = _oracle(orc, w, S.BF16, F, s)
    assert orc.blob_exceptions(blob_o) > 10000
    blob, _ = gpu_compress(w, S.BF16, 3.0, F, force_scale=s)
    assert np.array_equal(blob, blob_o)
    err, out = GpuBlob(blob).decode()
    assert err == 0 and np.array_equal(out, ref)
