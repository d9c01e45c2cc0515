"""GPU edge cases of the whole library path (compress on the device, blob byte-identical to the
oracle's, decode bit-identical): degenerate shapes, a matrix whose payload is empty, a constant
matrix, one huge row, and a zero row among normal ones; every GPU call repeated on the same
inputs gives the same bytes; and bad inputs to compress return the oracle's status."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import (GpuBlob, ep_mod, gpu_compress, gpu_quantize, gpu_row_lsq, gpu_row_sumsq,
                      log)

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


def test_every_call_is_deterministic():
    """Each GPU call run twice on the same inputs gives the same bytes: the quantiser's cosets,
    fields and histogram (integer atomics in any order), the fp64 row sums and LS terms (one
    lane per row, fixed order), the whole library compress (rate search, tables, tile encoder)
    with and without the per-row refinement, and the single and batched decodes."""
    import torch

    ep = ep_mod()
    log("determinism")
    w = S.workload_weights(2, 300, 1000, 0)             # ragged width, several tiles
    ss1, ss2 = gpu_row_sumsq(w, S.BF16), gpu_row_sumsq(w, S.BF16)
    assert np.array_equal(ss1.view(np.uint64), ss2.view(np.uint64))
    g = (1.0 / (np.sqrt(ss1 / 1000.0) * 0.3)).astype(np.float32)
    q1, q2 = gpu_quantize(w, S.BF16, g), gpu_quantize(w, S.BF16, g)
    for a, b in zip(q1, q2):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    assert q1[0] == 0
    l1, l2 = gpu_row_lsq(w, S.BF16, q1[1], q1[2]), gpu_row_lsq(w, S.BF16, q1[1], q1[2])
    assert np.array_equal(l1[0].view(np.uint64), l2[0].view(np.uint64))
    assert np.array_equal(l1[1], l2[1])
    for refine in (0, 5):
        b1, s1 = gpu_compress(w, S.BF16, 3.5, 8192, refine=refine)
        b2, s2 = gpu_compress(w, S.BF16, 3.5, 8192, refine=refine)
        assert s1 == s2 and np.array_equal(b1, b2)
    blob, _ = gpu_compress(w, S.BF16, 3.5, 8192)
    gb = GpuBlob(blob)
    e1, o1 = gb.decode()
    e2, o2 = gb.decode()
    assert e1 == 0 and e2 == 0 and np.array_equal(o1, o2)
    outs = [torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda") for _ in range(3)]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        assert ep.ep_decompress_batch([gb.d_blob] * 3, [gb.info] * 3, [gb.d_tab] * 3, outs,
                                      d_err) == 0
        torch.cuda.synchronize()
        assert int(d_err.item()) == 0
        for o in outs:
            got = o.cpu().numpy().view(np.uint16).reshape(300, gb.pitch())[:, :1000]
            assert np.array_equal(got, o1)


def _lib_status(w, dt, target, F, force_scale=0.0):
    ep = ep_mod()
    try:
        gpu_compress(w, dt, target, F, force_scale=force_scale)
    except ep.EPError as e:
        return e.status
    return 0


def test_compress_failures_match_oracle(orc):
    """Failure injection through the whole library compress: each bad input returns the status
    the oracle returns for it (non-finite input, target rate outside its range or NaN, a scale
    that pushes the lattice coordinates past the field range), and the library stays usable; a
    scale that gives a field more distinct values than the 2^12 slots of its table compresses
    on both sides, with escapes, to the same blob."""
    log("compress failures")
    w = S.workload_weights(2, 64, 1024, 0)
    nan_w, inf_w = w.copy(), w.copy()
    nan_w[5, 17] = 0x7FC0                                    # bf16 NaN
    inf_w[60, 1000] = 0xFF80                                 # bf16 -inf
    wide = S.iid_normal(512, 1024, seed=9)                   # 65536 vectors
    cases = [
        (nan_w, 3.0, 0.0, "nan input"),
        (inf_w, 3.0, 0.0, "inf input"),
        (w, 0.0005, 0.0, "target below range"),
        (w, 11.5, 0.0, "target above range"),
        (w, float("nan"), 0.0, "nan target"),
        (w, 3.0, 1e-7, "coordinates past the field range"),
    ]
    seen = set()
    for x, target, fs, what in cases:
        st_o = orc.compress(x, S.BF16, target, 8192, force_s=fs)[0]
        st_l = _lib_status(x, S.BF16, target, 8192, force_scale=fs)
        assert st_o != 0 and st_l == st_o, (what, st_l, st_o)
        seen.add(st_o)
    assert {orc.ERR_NONFINITE, orc.ERR_ARG, orc.ERR_RANGE} <= seen
    # more distinct values than a table's 2^12 slots is no failure: both sides escape them
    st_o, blob_o, _ = orc.compress(wide, S.BF16, 3.0, 8192, force_s=1.0 / 3000.0)
    assert st_o == 0 and orc.blob_exceptions(blob_o) > 0
    blob_l, _ = gpu_compress(wide, S.BF16, 3.0, 8192, force_scale=1.0 / 3000.0)
    assert np.array_equal(blob_l, blob_o)
    blob, _ = gpu_compress(w, S.BF16, 3.0, 8192)            # still works afterwards
    st, blob_o, _ = orc.compress(w, S.BF16, 3.0, 8192)
    assert st == 0 and np.array_equal(blob, blob_o)
