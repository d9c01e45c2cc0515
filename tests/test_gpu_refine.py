"""GPU parity of the per-row rate-distortion refinement: the per-row rate kernel
(ep_row_rates) against the oracle's row rates, and the library's refined compress (device
quantiser, LS terms, table build and rates; host selection) against the oracle's refined blob,
byte for byte.  Inputs: seeded synthetic weights (ep_synth)."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import dev, ep_mod, gpu_compress, host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key,R,C,s", [(2, 64, 1024, 0.2), (3, 37, 1032, 0.05),
                                       ("5b", 8, 16384, 0.02)])
def test_row_rates_match_oracle(orc, key, R, C, s):
    import torch

    log("row rates", key, R, C)
    ep = ep_mod()
    w = S.workload_weights(key, R, C)
    dt = S.WORKLOADS[key]["dtype"]
    st, cos, fld = orc.quantize(w, dt, orc.gains(orc.row_sumsq(w, dt), C, s))
    assert st == 0
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    assert st == 0
    # a model that lacks some of the values: the tables of a coarser quantisation
    st, cos2, fld2 = orc.quantize(w, dt, orc.gains(orc.row_sumsq(w, dt), C, 2 * s))
    st, lo2, n2, freq2 = orc.build_tables(orc.histogram(cos2, fld2))
    cost = orc.rate_costs()
    for (l_, n_, f_) in ((lo, n, freq), (lo2, n2, freq2)):
        want = orc.row_rates(cos, fld, R, C, l_, n_, f_, cost)
        d_tab = dev(ep.tables_struct(l_, n_, f_))
        d_rates = torch.zeros(R, dtype=torch.int64, device="cuda")
        assert ep.ep_row_rates(dev(cos), dev(fld), R, C, d_tab, dev(cost), d_rates) == 0
        torch.cuda.synchronize()
        assert np.array_equal(host(d_rates), want)


# (workload recipe, rows, cols, candidates)
CASES = [
    (2, 64, 1024, 5),
    (2, 96, 512, 9),
    (3, 64, 1024, 3),
    ("5a", 32, 2048, 5),
    ("5b", 32, 2048, 3),
    (1, 256, 256, 5),
    (4, 48, 3072, 5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-n{c[3]}")
def test_refined_compress_matches_oracle(orc, case):
    key, R, C, nc = case
    log("refined compress", case)
    wl = S.WORKLOADS[key]
    w = S.workload_weights(key, R, C)
    st, blob_o, s_o = orc.compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"],
                                   refine=nc)
    assert st == 0
    blob, s = gpu_compress(w, wl["dtype"], wl["target_bpp"], wl["tile_fields"], refine=nc)
    assert s == s_o
    assert blob.size == blob_o.size and np.array_equal(blob, blob_o)


def test_refined_compress_fp32_matches_oracle(orc):
    log("refined compress fp32")
    w = S.lognormal_rows(128, 512, seed=44, sigma=0.8, dtype=S.FP32)
    st, blob_o, _ = orc.compress(w, S.FP32, 3.0, 4096, refine=5)
    assert st == 0
    blob, _ = gpu_compress(w, S.FP32, 3.0, 4096, refine=5)
    assert np.array_equal(blob, blob_o)


def test_refine_high_level():
    import torch

    import entropy_coded_weight_ep_amd as ep

    log("refine high level")
    w = S.lognormal_rows(256, 1024, seed=45, sigma=0.8)
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    errs = {}
    for refine in (0, True):
        c = ep.compress(t, ep.LatticeRANSConfig(target_bpp=3.0, tile_fields=8192, refine=refine))
        r = ep.decompress(c)
        errs[refine] = ((r.float() - t.float()).norm() / t.float().norm()).item()
    assert errs[True] < errs[0]
    with pytest.raises(ep.EPError):
        ep.compress(t, ep.LatticeRANSConfig(target_bpp=3.0, refine=2))
