"""GPU parity with 128 rANS states per tile (two per wavefront lane) and at non-default rate-search
settings.

The coder and its word order are those of 64 states per tile with vector l + 64u of a tile owned
by state l + 64 (u mod 2) (design page "EntroPack lattice compression", *Encoding and
reconstruction*: rANS in independently decodable tiles); the oracle produces such blobs
(lanes=128) and the tests hold the library to them bit for bit: the decode of every workload
shape (ragged tiles, wide alphabets, all three tile sizes, both word layouts, batches), the device
tile encoder, and the library's compress, whose blob must equal the oracle's byte for byte.  The
rate-search settings of *Usage* (sample rows, bisection steps, the whole-tensor rate check) are
checked the same way."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, ep_mod, gpu_compress, gpu_encode_tiles, log

pytestmark = pytest.mark.gpu

DECODE_CASES = [
    (1, 256, 256),          # 4096-field tiles, J = 8 per lane, 4 per state
    (2, 512, 1024),         # J = 16
    (2, 200, 776),          # ragged last tile
    (3, 256, 1024),         # fp16, wide alphabet
    (4, 96, 3072),          # tiles span rows
    ("5a", 64, 2048),       # fp8, J = 32
    ("5b", 64, 2048),       # int8, J = 32, wide alphabet
    ("5b", 37, 1000),       # ragged, J = 32
    (1, 3, 8),              # one vector per row, a single ragged tile
]


def _blob(orc, key, R, C, target=None, lanes=128):
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    st, blob, s = orc.compress(w, wl["dtype"], target or wl["target_bpp"], wl["tile_fields"],
                               lanes=lanes)
    assert st == 0
    return w, blob


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_decode_128_lanes_matches_oracle(orc, case):
    key, R, C = case
    log("decode 128 lanes", case)
    w, blob = _blob(orc, key, R, C)
    gb = GpuBlob(blob)
    assert gb.info.lanes == 128
    err, out = gb.decode()
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0 and err == 0
    assert np.array_equal(out, ref)
    # the same tensor as the 64-lane blob of the same scale
    wl = S.WORKLOADS[key]
    st, b64, _ = orc.compress(w, wl["dtype"], 1.0, wl["tile_fields"],
                              force_s=orc.blob_fields(blob)["s"])
    err64, out64 = GpuBlob(b64).decode()
    assert err64 == 0 and np.array_equal(out64, out)


@pytest.mark.parametrize("flags", ["LINEAR", "RING", "RING_MIN"])
@pytest.mark.parametrize("case", [(2, 512, 1024, None), (3, 256, 1024, None),
                                  ("5b", 64, 2048, None), ("5b", 37, 1000, None),
                                  (2, 128, 1024, 11.0), (1, 256, 256, 8.0)],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-{c[3]}")
def test_decode_128_lanes_word_layouts(orc, case, flags):
    key, R, C, target = case
    log("decode 128 lanes layout", case, flags)
    ep = ep_mod()
    w, blob = _blob(orc, key, R, C, target=target)
    err, out = GpuBlob(blob).decode(flags=getattr(ep, "EP_DECODE_" + flags))
    st, ref, _, _ = orc.decompress(blob)
    assert st == 0 and err == 0
    assert np.array_equal(out, ref)


def test_decode_128_lanes_detects_corruption(orc):
    log("decode 128 lanes corrupt")
    w, blob = _blob(orc, 2, 256, 1024)
    info = GpuBlob(blob).info
    bad = blob.copy()
    bad[-64] ^= 0x5A                                  # a payload word of the last tile
    err, _ = GpuBlob(bad).decode()
    assert err & (1 << 7)
    bad = blob.copy()
    o = info.off_states + 4 * 100                     # a state of tile 0's second half
    bad[o] ^= 0x5A
    err, _ = GpuBlob(bad).decode()
    assert err & (1 << 7)


def test_decode_batch_128_lanes(orc):
    """A batch of 128-lane blobs decodes as each one alone; a batch mixing lane counts is refused
    before anything is launched."""
    import torch

    ep = ep_mod()
    blobs, refs = [], []
    for i, (key, R, C) in enumerate([(2, 96, 1024), (2, 200, 776), (4, 96, 3072), (2, 64, 512)]):
        w, b = _blob(orc, key, R, C)
        blobs.append(GpuBlob(b))
        refs.append(orc.decompress(b)[1])
    outs = [torch.zeros(gb.out_bytes(), dtype=torch.uint8, device="cuda") for gb in blobs]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_batch([g.d_blob for g in blobs], [g.info for g in blobs],
                                [g.d_tab for g in blobs], outs, d_err)
    assert st == 0
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0
    for gb, o, ref in zip(blobs, outs, refs):
        got = o.cpu().numpy().view(np.uint16).reshape(gb.info.rows, gb.pitch())[:, :gb.info.cols]
        assert np.array_equal(got, ref)
    w, b64 = _blob(orc, 2, 96, 1024, lanes=64)
    g64 = GpuBlob(b64)
    st = ep.ep_decompress_batch([blobs[0].d_blob, g64.d_blob], [blobs[0].info, g64.info],
                                [blobs[0].d_tab, g64.d_tab], outs[:2], d_err)
    assert st == ep.EP_ERR_ARG


@pytest.mark.parametrize("nv,F,spread", [(512, 4096, 3.0), (5000, 4096, 3.0), (100, 8192, 1.0),
                                         (3000, 16384, 8.0), (2500, 8192, 300.0)])
def test_gpu_encoder_128_lanes_matches_oracle(orc, nv, F, spread):
    """Narrow (byte-held) and wide fields, every tile size, ragged tiles."""
    ep = ep_mod()
    g = np.random.Generator(np.random.PCG64(nv + F))
    cos = (g.random(nv) < 0.4).astype(np.uint8)
    fld = np.rint(g.standard_normal(nv * 8) * spread).astype(np.int16)
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    assert st == 0
    st_o, woff_o, states_o, words_o = orc.encode_tiles(cos, fld, F, 128, 12, lo, n, freq)
    st, err, woff, maxw, states, words = gpu_encode_tiles(cos, fld, F,
                                                          ep.tables_struct(lo, n, freq),
                                                          lanes=128)
    assert st == 0 and err == 0 and st_o == 0
    assert np.array_equal(woff, woff_o)
    assert np.array_equal(states, states_o)
    assert np.array_equal(words, words_o)
    assert maxw == int(np.max(np.diff(woff_o.astype(np.int64))))


@pytest.mark.parametrize("case", [(1, 256, 256), (2, 256, 1024), (3, 128, 1024), (4, 64, 3072),
                                  ("5a", 32, 2048), ("5b", 32, 2048)],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_compress_128_lanes_blob_matches_oracle(orc, case):
    key, R, C = case
    log("compress 128 lanes", case)
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    st, blob_o, s_o = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"],
                                   lanes=128)
    assert st == 0
    blob, s = gpu_compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"], lanes=128)
    assert s == s_o
    assert blob.size == blob_o.size and np.array_equal(blob, blob_o)


@pytest.mark.parametrize("sample_rows,search_iters", [(32, 40), (1000, 40), (256, 7), (64, 0)])
def test_compress_search_settings_match_oracle(orc, sample_rows, search_iters):
    """Rate-search settings other than the defaults: the same scale and blob as the oracle's."""
    log("compress settings", sample_rows, search_iters)
    w = S.workload_weights(2, 600, 512)
    st, blob_o, s_o = orc.compress(w, S.BF16, 3.0, 8192, sample_rows=sample_rows,
                                   search_iters=search_iters)
    assert st == 0
    blob, s = gpu_compress(w, S.BF16, 3.0, 8192, sample_rows=sample_rows,
                           search_iters=search_iters)
    assert s == s_o and np.array_equal(blob, blob_o)


def test_compress_128_lanes_with_refinement(orc):
    w = S.workload_weights(2, 256, 1024)
    st, blob_o, s_o = orc.compress(w, S.BF16, 4.0, 8192, refine=5, lanes=128)
    assert st == 0
    blob, s = gpu_compress(w, S.BF16, 4.0, 8192, refine=5, lanes=128)
    assert s == s_o and np.array_equal(blob, blob_o)


def test_high_level_api_with_128_lanes(orc):
    import torch

    ep = ep_mod()
    w = S.workload_weights(2, 512, 1024)
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    cfg = ep.LatticeRANSConfig(target_bpp=4.0, tile_fields=8192, lanes=128)
    c = ep.compress(t, cfg)
    r = ep.decompress(c, cfg)
    torch.cuda.synchronize()
    assert c.info.lanes == 128
    assert r.shape == t.shape and r.dtype == t.dtype
    st, ref, _, _ = orc.decompress(c.blob)
    assert st == 0
    assert np.array_equal(r.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    with pytest.raises(ep.EPError):
        ep.compress(t, ep.LatticeRANSConfig(target_bpp=4.0, tile_fields=8192, lanes=96))


@pytest.mark.parametrize("check", [True, False])
def test_compress_rate_check_matches_oracle(orc, check):
    """An int8 tensor of heavy-tailed values (the 8192 x 28672 int8 recipe at 1024 x 4096), where
    the sampled estimate undershoots the tensor's: with the check the library raises the scale on
    whole-tensor estimates exactly as the oracle does; without it both keep the sampled scale."""
    log("compress rate check", check)
    _, _, q = S.laplace_pair(1024, 4096, seed=5)
    st, blob_o, s_o = orc.compress(q, S.INT8, 6.0, 16384, rate_check=int(check))
    assert st == 0
    blob, s = gpu_compress(q, S.INT8, 6.0, 16384, rate_check=check)
    assert s == s_o and np.array_equal(blob, blob_o)
    if check:
        assert 8.0 * blob.size / q.size <= 6.0
