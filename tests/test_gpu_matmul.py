"""GPU parity of the decode fused into its consumer product (EntroPack abstract: decoding during
inference, for prefill- and denoiser-shaped products; design page "EntroPack lattice
compression", *Encoding and reconstruction*: one fused GPU operation reconstructs the weights).

ep_decompress_matmul computes Y = X W^T with W decoded inside the kernel.  The oracle gives the
same product in fp64 from its own decode (oracle.decompress_matmul) together with
B = |X| |W|^T.  The library accumulates products of 16-bit values (exact in fp32) in fp32, in an
order of its own, so any element may differ from the exact sum by at most the recursive-summation
bound of cols + 16 terms: |Y - Y_ref| <= (cols + 16) 2^-24 B (2^-24 the fp32 unit roundoff; the
16 covers the partial sums of the workgroup's waves).  When each output is a single product
(unit rows of X) the result is exact, and it is checked bit for bit."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, dev, ep_mod, host, log

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _blob(orc, key, R, C, lanes=64, F=None, target=None):
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    st, blob, _ = orc.compress(w, wl["dtype"], target or wl["target_bpp"],
                               F or wl["tile_fields"], lanes=lanes)
    assert st == 0
    return w, blob


def _run(gb, xbits, m, expect_err=0):
    import torch

    ep = ep_mod()
    d_x = dev(xbits.view(np.uint16))
    d_y = torch.full((m, gb.info.rows), float("nan"), dtype=torch.float32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_matmul(gb.d_blob, gb.info, gb.d_tab, d_x, m, d_y, d_err)
    assert st == 0, st
    torch.cuda.synchronize()
    err = int(host(d_err)[0])
    assert err == expect_err, hex(err)
    return host(d_y).astype(np.float64)


def _check(orc, blob, xbits, Y):
    st, Yr, B = orc.decompress_matmul(blob, xbits)
    assert st == 0
    C = xbits.shape[1]
    tol = (C + 16) * U32 * B + 1e-30
    bad = np.abs(Y - Yr) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], Y[bad][:5], Yr[bad][:5], tol[bad][:5])


CASES = [
    # (workload, rows, cols, m, lanes, tile_fields)
    (2, 256, 4096, 16, 64, None),        # 8 tiles per 16 rows, aligned groups
    (2, 200, 776, 5, 64, None),          # ragged rows and tiles, groups straddle tiles, cols % 32
    (3, 512, 4096, 8, 64, None),         # fp16 with a wide alphabet
    (4, 96, 3072, 64, 64, None),         # denoiser width: 6 tiles per group, m = 64
    (2, 256, 1024, 17, 128, None),       # 128 rANS states per tile
    (1, 256, 256, 1, 64, 4096),          # 4096-field tiles, m = 1
    (2, 37, 1000, 33, 64, 4096),         # 4096-field tiles, ragged, unaligned groups
    (3, 64, 2048, 3, 128, 4096),         # fp16, 128 states, 4096-field tiles
    (2, 8200, 4096, 16, 64, None),       # two 16-row groups per workgroup, an odd group count
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-m{c[3]}-k{c[4]}")
def test_matmul_matches_oracle(orc, case):
    key, R, C, m, lanes, F = case
    log("decompress_matmul", case)
    _, blob = _blob(orc, key, R, C, lanes=lanes, F=F)
    gb = GpuBlob(blob)
    dt = S.WORKLOADS[key]["dtype"]
    xbits = S.iid_normal(m, C, 100 + m, sigma=1.0, dtype=dt)
    Y = _run(gb, xbits, m)
    _check(orc, blob, xbits, Y)


@pytest.mark.parametrize("key", [2, 3])
def test_matmul_unit_rows_exact(orc, key):
    """X rows with a single 1: each output is one decoded weight, so the result is exact."""
    R, C = (130, 1024) if key == 2 else (64, 4096)
    _, blob = _blob(orc, key, R, C)
    dt = S.WORKLOADS[key]["dtype"]
    st, wb, _, _ = orc.decompress(blob)
    assert st == 0
    W = S.container_to_float(wb, dt).astype(np.float64)
    ks = [0, 5, 31, 32, 500, C - 1]
    X = np.zeros((len(ks), C), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    Y = _run(GpuBlob(blob), S.cast_container(X, dt), len(ks))
    for i, k in enumerate(ks):
        assert np.array_equal(Y[i], W[:, k]), i


@pytest.mark.timeout(600)
@pytest.mark.parametrize("key,m", [(2, 16), (3, 8), (4, 64)])
def test_matmul_full_size(orc, key, m):
    """The full sizes of the prefill-shaped (14336 x 4096 fp16) and denoiser-shaped (3072^2
    bf16) matrices and of the 4096^2 bf16 one, in the launch configuration bench.py times."""
    wl = S.WORKLOADS[key]
    log("decompress_matmul full size", key, m)
    w = S.workload_weights(key)
    st, blob, _ = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"])
    assert st == 0
    del w
    xbits = S.iid_normal(m, wl["cols"], 200 + m, sigma=1.0, dtype=wl["dtype"])
    Y = _run(GpuBlob(blob), xbits, m)
    _check(orc, blob, xbits, Y)


def test_matmul_deterministic(orc):
    _, blob = _blob(orc, 2, 256, 4096)
    gb = GpuBlob(blob)
    xbits = S.iid_normal(16, 4096, 9, sigma=1.0, dtype=S.BF16)
    a = _run(gb, xbits, 16)
    b = _run(gb, xbits, 16)
    assert np.array_equal(a, b)


def test_matmul_refusals(orc):
    import torch

    ep = ep_mod()
    _, blob = _blob(orc, 2, 64, 1024)
    gb = GpuBlob(blob)
    d_x = torch.zeros((65, 1024), dtype=torch.bfloat16, device="cuda")
    d_y = torch.zeros((65, 64), dtype=torch.float32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    call = lambda g, x, m, y: ep.ep_decompress_matmul(g.d_blob, g.info, g.d_tab, x, m, y, d_err)
    assert call(gb, d_x, 0, d_y) == ep.EP_ERR_ARG
    assert call(gb, d_x, 65, d_y) == ep.EP_ERR_ARG
    xv = d_x.view(-1)[1:].view(torch.uint8)             # 2-byte offset: not 16-byte aligned
    assert call(gb, xv, 4, d_y) == ep.EP_ERR_ARG
    # containers other than bf16 / fp16
    _, b8 = _blob(orc, "5a", 32, 1024)
    assert call(GpuBlob(b8), d_x, 4, d_y) == ep.EP_ERR_DTYPE
    # rows wider than 4096, and 16384-field tiles
    _, bw = _blob(orc, 2, 16, 4104)
    assert call(GpuBlob(bw), d_x, 4, d_y) == ep.EP_ERR_SHAPE
    _, bt = _blob(orc, 2, 64, 1024, F=16384)
    assert call(GpuBlob(bt), d_x, 4, d_y) == ep.EP_ERR_SHAPE
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) == 0                     # nothing was launched


def test_matmul_detects_corruption(orc):
    _, blob = _blob(orc, 2, 128, 1024)
    bad = blob.copy()
    bad[-64] ^= 0x5A                                    # a payload word of the last tile
    xbits = S.iid_normal(4, 1024, 3, sigma=1.0, dtype=S.BF16)
    import torch

    ep = ep_mod()
    gb = GpuBlob(bad)
    d_y = torch.zeros((4, 128), dtype=torch.float32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_matmul(gb.d_blob, gb.info, gb.d_tab, dev(xbits.view(np.uint16)), 4,
                                 d_y, d_err)
    assert st == 0
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) & (1 << ep.EP_ERR_CORRUPT)


def test_high_level_decompress_matmul(orc):
    import torch

    ep = ep_mod()
    w = S.workload_weights(2, 256, 1024)
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    c = ep.compress(t, ep.LatticeRANSConfig(target_bpp=4.0, tile_fields=8192))
    xbits = S.iid_normal(12, 1024, 4, sigma=1.0, dtype=S.BF16)
    x = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).cuda()
    y = ep.decompress_matmul(c, x)
    torch.cuda.synchronize()
    assert y.shape == (12, 256) and y.dtype == torch.float32
    _check(orc, c.blob, xbits, host(y).astype(np.float64))
    with pytest.raises(ep.EPError):
        ep.decompress_matmul(c, x.float())


# ---- ep_decompress_matmul_batch: many blobs of one shape in one call ----------------------

def _weights(key, R, C, i):
    if key == 4:
        return S.workload_weights(4, R, C, index=i)
    if key == 3:
        return S.student_t_outliers(R, C, seed=60 + i)
    return S.lognormal_rows(R, C, seed=50 + i)


def _batch_run(gbs, xs, m, expect_err=0):
    import torch

    ep = ep_mod()
    d_xs = [dev(x.view(np.uint16)) for x in xs]
    d_ys = [torch.full((m, gb.info.rows), float("nan"), dtype=torch.float32, device="cuda")
            for gb in gbs]
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_decompress_matmul_batch([g.d_blob for g in gbs], [g.info for g in gbs],
                                       [g.d_tab for g in gbs], d_xs, m, d_ys, d_err)
    assert st == 0, st
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) == expect_err
    return [host(y).astype(np.float64) for y in d_ys]


BATCH_CASES = [
    # (workload, rows, cols, m, blobs, lanes)
    (4, 96, 3072, 16, 5, 64),            # denoiser width: 6 tiles per 16-row group
    (3, 64, 4096, 8, 3, 64),             # fp16 with a wide alphabet
    (2, 200, 776, 5, 4, 128),            # ragged rows and tiles, 128 states per tile
    (2, 48, 1024, 3, 35, 64),            # 35 blobs: two launches
]


@pytest.mark.parametrize("case", BATCH_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-m{c[3]}-n{c[4]}-k{c[5]}")
def test_matmul_batch_matches_oracle(orc, case):
    key, R, C, m, n, lanes = case
    log("decompress_matmul_batch", case)
    wl = S.WORKLOADS[key]
    dt = wl["dtype"]
    blobs, xs = [], []
    for i in range(n):
        st, blob, _ = orc.compress(_weights(key, R, C, i), dt, wl["target_bpp"],
                                   wl["tile_fields"], lanes=lanes)
        assert st == 0
        blobs.append(blob)
        xs.append(S.iid_normal(m, C, 300 + i, sigma=1.0, dtype=dt))
    Ys = _batch_run([GpuBlob(b) for b in blobs], xs, m)
    for blob, x, Y in zip(blobs, xs, Ys):
        _check(orc, blob, x, Y)


def test_matmul_batch_deterministic_and_refusals(orc):
    import torch

    ep = ep_mod()
    gbs = [GpuBlob(orc.compress(S.lognormal_rows(64, 1024, seed=70 + i), S.BF16, 4.0, 8192)[1])
           for i in range(3)]
    xs = [S.iid_normal(4, 1024, 80 + i, sigma=1.0, dtype=S.BF16) for i in range(3)]
    a = _batch_run(gbs, xs, 4)
    b = _batch_run(gbs, xs, 4)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    d_x = dev(xs[0].view(np.uint16))
    d_y = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call(gl, m=4):
        return ep.ep_decompress_matmul_batch([g.d_blob for g in gl], [g.info for g in gl],
                                             [g.d_tab for g in gl], [d_x] * len(gl), m,
                                             [d_y] * len(gl), d_err)

    assert call([]) == ep.EP_ERR_ARG                      # no blobs
    assert call(gbs, m=65) == ep.EP_ERR_ARG
    other_rows = GpuBlob(orc.compress(S.lognormal_rows(48, 1024, seed=9), S.BF16, 4.0, 8192)[1])
    assert call([gbs[0], other_rows]) == ep.EP_ERR_ARG    # shapes differ
    other_k = GpuBlob(orc.compress(S.lognormal_rows(64, 1024, seed=9), S.BF16, 4.0, 8192,
                                   lanes=128)[1])
    assert call([gbs[0], other_k]) == ep.EP_ERR_ARG       # states per tile differ
    fp16 = GpuBlob(orc.compress(S.student_t_outliers(64, 1024, seed=9), S.FP16, 4.0, 8192)[1])
    assert call([gbs[0], fp16]) == ep.EP_ERR_ARG          # containers differ
    torch.cuda.synchronize()
    assert int(host(d_err)[0]) == 0                       # nothing was launched


@pytest.mark.timeout(900)
def test_matmul_batch_full_size_denoiser(orc):
    """All 64 matrices of the 3072 x 3072 bf16 denoiser batch, m = 16, in one call (two launches
    of 32 blobs): each product within the bound of the oracle's fp64 product of its decode."""
    from concurrent.futures import ThreadPoolExecutor

    from gpu_util import gpu_compress

    wl = S.WORKLOADS[4]
    R, C, dt, F, nb, m = wl["rows"], wl["cols"], wl["dtype"], wl["tile_fields"], wl["batch"], 16
    log("library compress of the 64 denoiser matrices")
    blobs = [gpu_compress(S.workload_weights(4, index=i), dt, wl["target_bpp"], F)[0]
             for i in range(nb)]
    xs = [S.iid_normal(m, C, 400 + i, sigma=1.0, dtype=dt) for i in range(nb)]
    log("batched decompress_matmul")
    Ys = _batch_run([GpuBlob(b) for b in blobs], xs, m)
    log("oracle products (threaded) and compare")
    with ThreadPoolExecutor(16) as ex:
        refs = list(ex.map(lambda i: orc.decompress_matmul(blobs[i], xs[i]), range(nb)))
    for i, (st, Yr, B) in enumerate(refs):
        assert st == 0
        tol = (C + 16) * U32 * B + 1e-30
        assert not (np.abs(Ys[i] - Yr) > tol).any(), f"matrix {i}"


def test_high_level_decompress_matmul_batch(orc):
    import torch

    ep = ep_mod()
    cs, xbs, xs = [], [], []
    for i in range(3):
        w = S.lognormal_rows(128, 1024, seed=90 + i)
        t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
        cs.append(ep.compress(t, ep.LatticeRANSConfig(target_bpp=4.0, tile_fields=8192)))
        xb = S.iid_normal(6, 1024, 95 + i, sigma=1.0, dtype=S.BF16)
        xbs.append(xb)
        xs.append(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda())
    ys = ep.decompress_matmul_batch(cs, xs)
    torch.cuda.synchronize()
    assert len(ys) == 3
    for c, xb, y in zip(cs, xbs, ys):
        assert y.shape == (6, 128) and y.dtype == torch.float32
        _check(orc, c.blob, xb, host(y).astype(np.float64))
    with pytest.raises(ep.EPError):
        ep.decompress_matmul_batch(cs, xs[:2])
    with pytest.raises(ep.EPError):
        ep.decompress_matmul_batch(cs, [xs[0], xs[1], xs[2][:3]])
