"""GPU parity at the full sizes of the five workloads, every element compared, in the launch
configuration that bench.py times.

For each workload the oracle compresses the full synthetic tensor; the library's compress must
produce the same blob byte for byte, and the GPU decode of that blob must equal the oracle's
decode element for element (the coder is lossless, design page "EntroPack lattice compression",
*Encoding and reconstruction*, so the decoded cosets and fields -- and through them the output --
are fixed exactly).  The oracle's tile-range decode runs on host threads over disjoint tile
ranges.  The 64-matrix denoiser batch goes through ep_decompress_batch, the call bench.py times
for that workload, all 64 blobs in one call."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, ep_mod, gpu_compress, host, log

pytestmark = pytest.mark.gpu

THREADS = 16


def oracle_decode_threaded(orc, blob: np.ndarray) -> np.ndarray:
    """The oracle's decode of every tile, split over host threads (ctypes releases the GIL);
    each thread writes only its own tiles' elements of the shared output."""
    info = orc.blob_fields(blob)
    R, C, T = info["rows"], info["cols"], info["tiles"]
    out = np.zeros((R, C), orc.bits_dtype(info["dtype"]))
    bounds = np.linspace(0, T, min(THREADS, T) + 1).astype(np.int64)

    def run(i):
        return orc.lib().or_decompress(orc._p(blob), blob.size, int(bounds[i]),
                                       int(bounds[i + 1]), orc._p(out), None, None)

    with ThreadPoolExecutor(THREADS) as ex:
        sts = list(ex.map(run, range(len(bounds) - 1)))
    assert all(s == 0 for s in sts), sts
    return out


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("key", [2, 3, "5a", "5b"])
def test_full_size_workload(orc, key):
    wl = S.WORKLOADS[key]
    R, C, dt, F = wl["rows"], wl["cols"], wl["dtype"], wl["tile_fields"]
    log(f"full size {key}: {wl['name']}: generate")
    w = S.workload_weights(key)
    log("oracle compress")
    st, blob_o, s_o = orc.compress(w, dt, wl["target_bpp"], F)
    assert st == 0
    info = orc.blob_fields(blob_o)
    log(f"  s={s_o} actual_bpp={8 * blob_o.size / w.size:.4f} tiles={info['tiles']}")
    log("library compress")
    blob, s = gpu_compress(w, dt, wl["target_bpp"], F)
    assert s == s_o
    assert blob.size == blob_o.size and np.array_equal(blob, blob_o)
    # the stored rate: at most the target (the whole-tensor check), within 3% of it
    bpp = 8.0 * blob.size / w.size
    assert 0.97 * wl["target_bpp"] <= bpp <= wl["target_bpp"], bpp
    del blob, w
    log("gpu decode")
    err, out = GpuBlob(blob_o).decode()
    assert err == 0
    log("oracle decode (every tile, threaded)")
    ref = oracle_decode_threaded(orc, blob_o)
    bad = np.flatnonzero(out.reshape(-1) != ref.reshape(-1))
    assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:8]}"


@pytest.mark.timeout(1200)
def test_full_size_denoiser_batch(orc):
    """All 64 matrices of 3072 x 3072: blobs byte-identical to the oracle's, and one
    ep_decompress_batch call (launches of up to 32 blobs) decoding all of them exactly."""
    import torch

    ep = ep_mod()
    wl = S.WORKLOADS[4]
    R, C, dt, F, nb = wl["rows"], wl["cols"], wl["dtype"], wl["tile_fields"], wl["batch"]
    log("generate + oracle compress 64 matrices (threaded)")

    def make(i):
        w = S.workload_weights(4, index=i)
        st, b, s = orc.compress(w, dt, wl["target_bpp"], F)
        assert st == 0
        return w, b, s

    with ThreadPoolExecutor(THREADS) as ex:
        made = list(ex.map(make, range(nb)))
    log("library compress 64 matrices")
    for i, (w, b, s) in enumerate(made):
        blob, sl = gpu_compress(w, dt, wl["target_bpp"], F)
        assert sl == s and np.array_equal(blob, b), i
    blobs = [GpuBlob(b) for _, b, _ in made]
    outs = [torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda") for gb in blobs]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    log("batched decode of 64 blobs")
    st = ep.ep_decompress_batch([gb.d_blob for gb in blobs], [gb.info for gb in blobs],
                                [gb.d_tab for gb in blobs], outs, d_err)
    assert st == 0
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) == 0
    log("oracle decode of 64 blobs (threaded) and compare")
    refs = []
    with ThreadPoolExecutor(THREADS) as ex:
        refs = list(ex.map(lambda m: orc.decompress(m[1])[1], made))
    for i in range(nb):
        got = host(outs[i]).view(np.uint16).reshape(R, C)
        assert np.array_equal(got, refs[i]), f"matrix {i} differs"
