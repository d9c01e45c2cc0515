"""GPU parity of the device side of the rate search: the table build of a device histogram
(ep_build_tables_gpu) against the oracle's table build, and the per-candidate size estimate
(ep_estimate_bpp_gpu) against the oracle's estimate, both bit for bit.

Histograms come from the oracle's quantiser on seeded synthetic weights, from seeded random
fields of several spreads, and from hand-built counts that reach each branch of the
normalisation rule: a deficit, an excess taken over several rounds, ties, a single value, the
widest span, and too many distinct values.
"""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import dev, ep_mod, host, log

pytestmark = pytest.mark.gpu

ERR_ALPHABET = 6


def gpu_tables(counts):
    """-> (err word, lo, n, freq[17, 65536]) of ep_build_tables_gpu on a device copy."""
    import torch

    ep = ep_mod()
    d_hist = dev(np.ascontiguousarray(counts.astype(np.uint32)))
    d_out = torch.zeros(ep.TABLES_BYTES, dtype=torch.uint8, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert ep.ep_build_tables_gpu(d_hist, d_out, d_err) == 0
    torch.cuda.synchronize()
    out = host(d_out)
    lo = out[:68].view(np.int32)
    n = out[68:136].view(np.uint32)
    freq = out[136:].view(np.uint16).reshape(17, 65536)
    return int(host(d_err)[0]), lo, n, freq


def check_tables(orc, counts):
    st_o, lo_o, n_o, freq_o = orc.build_tables(counts)
    err, lo, n, freq = gpu_tables(counts)
    if st_o != 0:
        assert st_o == orc.ERR_ALPHABET and err & (1 << ERR_ALPHABET)
        return
    assert err == 0
    assert np.array_equal(lo, lo_o) and np.array_equal(n, n_o)
    for t in range(17):
        assert np.array_equal(freq[t, :n[t]], freq_o[t, :n_o[t]]), t


@pytest.mark.parametrize("seed", range(6))
def test_build_tables_gpu_random_fields(orc, seed):
    log("tables random", seed)
    g = np.random.Generator(np.random.PCG64(100 + seed))
    nv = int(g.integers(100, 20000))
    cos = (g.random(nv) < 0.3).astype(np.uint8)
    spread = [0.5, 2.0, 10.0, 60.0, 300.0, 1500.0][seed]
    fld = np.clip(np.rint(g.standard_t(3, nv * 8) * spread), -32767, 32767).astype(np.int16)
    check_tables(orc, orc.histogram(cos, fld))


@pytest.mark.parametrize("key,R,C,s", [(2, 256, 4096, 0.3), (3, 128, 4096, 0.01),
                                       ("5b", 64, 16384, 0.05), ("5a", 64, 8192, 2.0)])
def test_build_tables_gpu_quantised(orc, key, R, C, s):
    log("tables quantised", key, s)
    w = S.workload_weights(key, R, C)
    dt = S.WORKLOADS[key]["dtype"]
    st, cos, fld = orc.quantize(w, dt, orc.gains(orc.row_sumsq(w, dt), C, s))
    assert st == 0
    check_tables(orc, orc.histogram(cos, fld))


def test_build_tables_gpu_branches(orc):
    log("tables branches")
    c = np.zeros((17, 65536), np.uint64)
    c[0, 32768] = 7
    c[0, 32769] = 7                         # tie on the deficit: lowest index takes it
    # excess over four rounds: 4000 singletons and four equal heavy values
    c[1, 1000:5000] = 1
    c[1, [6000, 6001, 7000, 9000]] = 250000
    # a single value (frequency 2^P)
    c[2, 40000] = 123
    # the widest span: values at both ends of the int16 range, nothing between
    c[3, 1] = 5
    c[3, 65535] = 9
    # equal frequencies everywhere after the floor, with a small deficit
    c[4, 30000:30003] = 1
    # an excess on equal largest frequencies (lowest index gives first)
    c[5, 100:3000] = 1
    c[5, 50000] = 40000
    c[5, 50001] = 40000
    check_tables(orc, c)


def test_build_tables_gpu_alphabet_error(orc):
    log("tables alphabet")
    c = np.zeros((17, 65536), np.uint64)
    c[0, 32768] = 10
    c[7, 32768 - 3000:32768 + 1097] = 1     # 4097 distinct values
    check_tables(orc, c)


@pytest.mark.parametrize("key,R,C,F,s", [(2, 600, 512, 4096, 0.05), (2, 600, 512, 4096, 1.0),
                                         (3, 700, 1024, 8192, 0.01),
                                         ("5b", 300, 2048, 16384, 0.3),
                                         (1, 256, 256, 4096, 0.5)])
def test_estimate_gpu_matches_oracle(orc, key, R, C, F, s):
    import torch

    log("estimate", key, s)
    ep = ep_mod()
    w = S.workload_weights(key, R, C)
    dt = S.WORKLOADS[key]["dtype"]
    ns = min(R, 256)
    sel = (np.arange(ns) * R) // ns
    g = orc.gains(orc.row_sumsq(w, dt), C, s)
    st, cos, fld = orc.quantize(w, dt, g, row_sel=sel)
    assert st == 0
    d_hist = dev(orc.histogram(cos, fld).astype(np.uint32))
    wsb = ep.ep_estimate_workspace_bytes()
    d_ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    got = ep.ep_estimate_bpp_gpu(d_hist, R, C, ns, F, d_ws, wsb)
    want = orc.estimate_bpp(w, dt, F, s)
    assert np.float64(got).view(np.uint64) == np.float64(want).view(np.uint64), (got, want)
    # a second call on the same workspace gives the same value
    assert ep.ep_estimate_bpp_gpu(d_hist, R, C, ns, F, d_ws, wsb) == got


def test_estimate_gpu_alphabet_and_arguments(orc):
    import torch

    log("estimate errors")
    ep = ep_mod()
    c = np.zeros((17, 65536), np.uint32)
    c[0, 32768] = 10
    c[7, 32768 - 3000:32768 + 1097] = 1
    wsb = ep.ep_estimate_workspace_bytes()
    d_ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    assert ep.ep_estimate_bpp_gpu(dev(c), 64, 64, 64, 4096, d_ws, wsb) == float("inf")
    assert ep.ep_estimate_bpp_gpu(dev(c), 64, 64, 64, 4096, d_ws, wsb - 1) == float("inf")
