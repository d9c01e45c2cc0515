"""GPU edge cases of the whole library path (compress on the device, blob byte-identical to the
oracle's, decode bit-identical): degenerate shapes, a matrix whose payload is empty, a constant
matrix, one huge row, and a zero row among normal ones."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, gpu_compress, log

pytestmark = pytest.mark.gpu


def _roundtrip(orc, w, dt, target, F):
    blob, s = gpu_compress(w, dt, target, F)
    st, blob_o, s_o = orc.compress(w, dt, target, F)
    assert st == 0 and s == s_o
    assert np.array_equal(blob, blob_o)
    err, out = GpuBlob(blob).decode()
    st, ref, _, _ = orc.decompress(blob_o)
    assert err == 0 and st == 0 and np.array_equal(out, ref)
    return blob


@pytest.mark.parametrize("shape", [(1, 1), (1, 7), (3, 9), (1, 8), (2, 4096), (1, 80000)],
                         ids=str)
def test_degenerate_shapes(orc, shape):
    log("edge shape", shape)
    R, C = shape
    w = S.lognormal_rows(R, C, seed=90 + C)
    _roundtrip(orc, w, S.BF16, 4.0, 4096)


def test_all_zero_matrix_has_no_payload(orc):
    log("edge zeros")
    w = np.zeros((64, 512), np.uint16)
    blob = _roundtrip(orc, w, S.BF16, 3.0, 8192)
    assert orc.blob_fields(blob)["payload_words"] == 0


def test_constant_matrix(orc):
    log("edge constant")
    w = np.full((40, 264), S.cast_container(np.array([0.0123], np.float32), S.FP16)[0], np.uint16)
    _roundtrip(orc, w, S.FP16, 2.0, 4096)


def test_zero_rows_among_others(orc):
    log("edge zero rows")
    w = S.lognormal_rows(50, 1024, seed=91)
    w[[0, 7, 49]] = 0
    _roundtrip(orc, w, S.BF16, 4.0, 8192)
