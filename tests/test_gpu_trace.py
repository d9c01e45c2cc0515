"""The traced decode (ep_decompress_traced): the decoder with a per-tile clock record of its
phases.  It must decode exactly as ep_decompress does (the tiles are the same lossless rANS
tiles, design page "EntroPack lattice compression", *Encoding and reconstruction*), and every
tile's record must be complete and ordered: start, landed, coset phase, then for each field phase
its barrier and its end, then the end-of-tile check."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, ep_mod, host, log

pytestmark = pytest.mark.gpu

CASES = [
    (2, 256, 1024, 64, None),        # bf16, 16 vectors per lane
    (2, 200, 776, 64, None),         # ragged last tile
    (2, 256, 1024, 128, None),       # two states per lane
    (1, 256, 256, 64, 4096),         # 8 vectors per lane
    ("5a", 64, 2048, 64, None),      # fp8, 32 vectors per lane
    ("5a", 37, 1000, 128, None),     # fp8, ragged, two states per lane
    (3, 64, 1024, 64, 8192),         # a wide alphabet, carried by a bf16 blob of the fp16 recipe
]


def _blob(orc, key, R, C, lanes, F, dtype=None):
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    dt = dtype or wl["dtype"]
    if dtype is not None and dtype != wl["dtype"]:
        w = S.cast_container(S.container_to_float(w, wl["dtype"]), dtype)
    st, blob, _ = orc.compress(w, dt, wl["target_bpp"], F or wl["tile_fields"], lanes=lanes)
    assert st == 0
    return blob


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-k{c[3]}")
def test_traced_decode_matches_and_records_every_tile(orc, case):
    import torch

    key, R, C, lanes, F = case
    log("traced decode", case)
    dtype = S.BF16 if key == 3 else None
    blob = _blob(orc, key, R, C, lanes, F, dtype)
    ep = ep_mod()
    gb = GpuBlob(blob)
    err_ref, ref = gb.decode()
    assert err_ref == 0
    T = gb.info.tiles
    d_out = torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_st = torch.zeros(T * ep.EP_TRACE_STAMPS, dtype=torch.int64, device="cuda")
    st = ep.ep_decompress_traced(gb.d_blob, gb.info, gb.d_tab, d_out, d_err, d_st)
    assert st == 0
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) == 0
    npdt = {1: np.uint16, 3: np.uint8}[gb.info.dtype]
    got = host(d_out).view(npdt).reshape(gb.info.rows, gb.pitch())[:, :gb.info.cols]
    assert np.array_equal(got, ref)
    a = host(d_st).reshape(T, ep.EP_TRACE_STAMPS)
    assert (a > 0).all()
    assert (np.diff(a, axis=1) >= 0).all()


def test_traced_decode_refusals(orc):
    import torch

    ep = ep_mod()
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    blob = _blob(orc, 3, 64, 1024, 64, None)             # fp16: not instantiated with the trace
    gb = GpuBlob(blob)
    d_out = torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda")
    d_st = torch.zeros(gb.info.tiles * ep.EP_TRACE_STAMPS + 1, dtype=torch.int64, device="cuda")
    assert ep.ep_decompress_traced(gb.d_blob, gb.info, gb.d_tab, d_out, d_err, d_st) == \
        ep.EP_ERR_VERSION
    gb2 = GpuBlob(_blob(orc, 2, 64, 1024, 64, None))
    d_out2 = torch.zeros(gb2.out_bytes(), dtype=torch.uint8, device="cuda")
    mis = d_st.view(torch.uint8)[4:]                       # 4-byte offset: not 8-byte aligned
    assert ep.ep_decompress_traced(gb2.d_blob, gb2.info, gb2.d_tab, d_out2, d_err, mis) == \
        ep.EP_ERR_ARG
    assert ep.ep_decompress_traced(gb2.d_blob, gb2.info, gb2.d_tab, d_out2, d_err, None) == \
        ep.EP_ERR_ARG
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) == 0
