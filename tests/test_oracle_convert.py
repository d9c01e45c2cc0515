"""Pins for the oracle's container conversions (EntroPack abstract: BF16, FP16, FP8 and INT8
containers; design page, "Encoding and reconstruction": the result keeps the input's dtype).

The oracle rounds from the definition (quantum of the binade, rint, then overflow); these tests
check it against independent library routines: torch's CPU casts for bf16 / fp16 / fp8 e4m3fn
and numpy rint + clip for int8, over every fp32 bit pattern whose low 12 bits come from a set
that straddles every rounding boundary of the three float formats (2^20 x 8 patterns).
"""

import numpy as np
import pytest
import torch

import ep_synth as S

LOW12 = np.array([0x000, 0x001, 0x3FF, 0x7FF, 0x800, 0x801, 0xC00, 0xFFF], np.uint32)


def structured_patterns():
    hi = np.arange(1 << 20, dtype=np.uint32) << 12
    return (hi[:, None] | LOW12[None, :]).reshape(-1)


@pytest.fixture(scope="module")
def pats():
    return structured_patterns().view(np.float32)


def _torch_cast(x, dt):
    t = torch.from_numpy(x)
    if dt == S.BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dt == S.FP16:
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("dt", [S.BF16, S.FP16])
def test_narrow_ieee_formats_match_torch(orc, pats, dt):
    got = orc.narrow(pats, dt)
    ref = _torch_cast(pats, dt)
    fin = ~np.isnan(pats)
    assert np.array_equal(got[fin], ref[fin])
    # NaN stays NaN
    back = S.container_to_float(got[~fin][:1000], dt)
    assert np.all(np.isnan(back))


def test_narrow_fp8_matches_torch_in_range_and_saturates(orc, pats):
    got = orc.narrow(pats, S.FP8)
    ref = _torch_cast(pats, S.FP8)
    with np.errstate(invalid="ignore"):
        a = np.abs(pats.astype(np.float64))
    # torch's cast is non-saturating; where the RNE result is representable both must agree
    inr = (~np.isnan(pats)) & (a < 464.0)
    assert np.array_equal(got[inr], ref[inr])
    # values whose rounding exceeds 448 saturate to +-448 (0x7E / 0xFE), infinities included
    big = (~np.isnan(pats)) & (a >= 464.0)
    sign = np.signbit(pats[big])
    assert np.all(got[big] == np.where(sign, 0xFE, 0x7E))
    # the tie between 448 and 480 rounds to even (448); just above it still saturates
    assert orc.narrow(np.array([464.0, -464.0, 463.99, 1e30], np.float32), S.FP8).tolist() == \
        [0x7E, 0xFE, 0x7E, 0x7E]
    # the subnormal step is 2^-9
    assert orc.narrow(np.array([2.0 ** -9, 2.0 ** -10, 1.5 * 2 ** -10], np.float32), S.FP8).tolist() == \
        [1, 0, 1]  # 2^-10 ties to even (0); 0.75 * 2^-9 rounds up


def test_narrow_int8_matches_numpy(orc, pats):
    got = orc.narrow(pats, S.INT8)
    with np.errstate(invalid="ignore"):
        x = pats.astype(np.float64)
    fin = ~np.isnan(x)
    ref = np.clip(np.rint(x[fin]), -128, 127).astype(np.int8)
    assert np.array_equal(got[fin], ref)
    assert np.all(got[~fin] == 0)


@pytest.mark.parametrize("dt", [S.BF16, S.FP16, S.FP8, S.INT8])
def test_widen_every_container_pattern(orc, dt):
    if dt in (S.BF16, S.FP16):
        bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    elif dt == S.FP8:
        bits = np.arange(256, dtype=np.uint32).astype(np.uint8)
    else:
        bits = np.arange(-128, 128).astype(np.int8)
    got = orc.widen(bits, dt)
    ref = S.container_to_float(bits, dt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


@pytest.mark.parametrize("dt", [S.BF16, S.FP16, S.FP8, S.INT8])
def test_roundtrip_every_container_value(orc, dt):
    """narrow(widen(b)) == b for every finite container value (no double rounding)."""
    if dt in (S.BF16, S.FP16):
        bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    elif dt == S.FP8:
        bits = np.arange(256, dtype=np.uint32).astype(np.uint8)
    else:
        bits = np.arange(-128, 128).astype(np.int8)
    vals = orc.widen(bits, dt)
    fin = np.isfinite(vals)
    back = orc.narrow(vals[fin], dt)
    assert np.array_equal(back.view(bits.dtype), bits[fin])


@pytest.mark.slow
@pytest.mark.parametrize("dt", [S.BF16, S.FP16, S.FP8])
def test_narrow_exhaustive_all_fp32(orc, dt):
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        x = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32).view(np.float32)
        got = orc.narrow(x, dt)
        ref = _torch_cast(x, dt)
        ok = ~np.isnan(x)
        if dt == S.FP8:
            ok &= np.abs(x.astype(np.float64)) < 464.0
        assert np.array_equal(got[ok], ref[ok])


def test_fp32_container_keeps_every_value(orc, pats):
    """The fp32 container (a reading beyond the abstract's list) stores the fp32 value itself:
    widening and narrowing are the identity on every non-NaN pattern, subnormals and infinities
    included; NaN stays NaN."""
    bits = pats.view(np.uint32)
    fin = ~np.isnan(pats)
    got = orc.widen(bits, S.FP32)
    assert np.array_equal(got[fin].view(np.uint32), bits[fin])
    assert np.all(np.isnan(got[~fin]))
    back = orc.narrow(pats, S.FP32)
    assert back.dtype == np.uint32
    assert np.array_equal(back[fin], bits[fin])
    assert np.all(np.isnan(back[~fin][:1000].view(np.float32)))
