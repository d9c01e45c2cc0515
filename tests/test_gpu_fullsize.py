"""GPU parity at the full sizes of the five workloads, in the launch configuration that bench.py
times (one ep_decompress per matrix).

For each workload the oracle compresses the full synthetic tensor; the library's compress must
produce the same blob byte for byte, and the GPU decode of the oracle's blob must equal the
oracle's decode (every element for the workloads the oracle decodes in seconds; sampled tiles --
first, middle and last -- for the two 8192 x 28672 tensors)."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, gpu_compress, log

pytestmark = pytest.mark.gpu

CASES = [(2, 0), (3, 0), (4, 0), (4, 63), ("5a", 0), ("5b", 0)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_full_size_workload(orc, case):
    key, index = case
    wl = S.WORKLOADS[key]
    R, C, dt, F = wl["rows"], wl["cols"], wl["dtype"], wl["tile_fields"]
    log(f"full size {key}/{index}: {wl['name']}: generate")
    w = S.workload_weights(key, index=index)
    log("oracle compress")
    st, blob_o, s_o = orc.compress(w, dt, wl["target_bpp"], F)
    assert st == 0
    info = orc.blob_fields(blob_o)
    log(f"  s={s_o} actual_bpp={8 * blob_o.size / w.size:.4f} tiles={info['tiles']}")
    log("library compress")
    blob, s = gpu_compress(w, dt, wl["target_bpp"], F)
    assert s == s_o
    assert blob.size == blob_o.size and np.array_equal(blob, blob_o)
    log("gpu decode")
    gb = GpuBlob(blob_o)
    err, out = gb.decode()
    assert err == 0
    T = info["tiles"]
    V = F // 8
    if R * C <= 60_000_000:
        log("oracle decode (all tiles)")
        st, ref, _, _ = orc.decompress(blob_o)
        assert st == 0 and np.array_equal(out, ref)
    else:
        picks = [(0, 3), (T // 2 - 1, T // 2 + 2), (T - 3, T)]
        for t0, t1 in picks:
            log(f"oracle decode tiles [{t0}, {t1})")
            st, ref, _, _ = orc.decompress(blob_o, t0, t1)
            assert st == 0
            e0, e1 = t0 * V * 8, min(t1 * V, R * C // 8) * 8
            assert np.array_equal(out.reshape(-1)[e0:e1], ref.reshape(-1)[e0:e1])
    del out
