"""GPU parity of the device tile encoder (ep_encode_tiles_gpu) with the oracle's tile encoder:
tile offsets, final states and the word stream compared bit for bit, and the largest tile word
count against the oracle's offsets.

Symbols come from the oracle's E8 quantiser on seeded synthetic weights (the encoder sees only
cosets and fields), at scales that give small alphabets (tables in LDS) and wide ones (more
than 16384 packed table entries: tables read from global memory), in every tile size, with
ragged last tiles and tiles of a single vector.
"""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import ep_mod, gpu_encode_tiles, log

pytestmark = pytest.mark.gpu

ERR_ALPHABET, ERR_CAPACITY, ERR_ARG = 6, 10, 1


def _symbols(orc, key, R, C, s):
    w = S.workload_weights(key, R, C)
    dt = S.WORKLOADS[key]["dtype"]
    g = orc.gains(orc.row_sumsq(w, dt), C, s)
    st, cos, fld = orc.quantize(w, dt, g)
    assert st == 0
    return cos, fld


def _tables(orc, cos, fld):
    st, lo, n, freq = orc.build_tables(orc.histogram(cos, fld))
    assert st == 0
    return lo, n, freq


def _check(orc, cos, fld, F, lo, n, freq):
    ep = ep_mod()
    st_o, woff_o, states_o, words_o = orc.encode_tiles(cos, fld, F, 64, 12, lo, n, freq)
    assert st_o == 0
    st, err, woff, mx, states, words = gpu_encode_tiles(cos, fld, F, ep.tables_struct(lo, n, freq))
    assert st == 0 and err == 0, (st, err)
    assert np.array_equal(woff, woff_o)
    assert mx == int(np.diff(woff_o.astype(np.int64)).max())
    assert np.array_equal(states, states_o)
    assert np.array_equal(words, words_o)
    return int(n.sum())


# (workload recipe, rows, cols, scale s, tile fields)
CASES = [
    (2, 37, 1032, 0.3, 4096),       # 8 vectors a lane, 9.3 tiles
    (2, 64, 4096, 0.05, 8192),      # 16 a lane, 32 whole tiles
    ("5b", 9, 16392, 0.05, 16384),  # 32 a lane, last tile of 9 vectors
    (1, 3, 8, 0.3, 4096),           # three vectors
    (3, 24, 4096, 0.01, 8192),      # wide alphabet: tables in global memory
    (3, 40, 4104, 0.003, 16384),    # wider still, 32 a lane
    ("5b", 16, 16384, 0.01, 4096),  # wide, 8 a lane
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-s{c[3]}-F{c[4]}")
def test_encode_tiles_matches_oracle(orc, case):
    key, R, C, s, F = case
    log("encode", case)
    cos, fld = _symbols(orc, key, R, C, s)
    lo, n, freq = _tables(orc, cos, fld)
    n_ent = _check(orc, cos, fld, F, lo, n, freq)
    if s <= 0.01:
        assert n_ent > 16384          # the case exercises the global-memory table path


def test_encode_tiles_single_symbol_tables(orc):
    # all-zero symbols: every table has one symbol of frequency 2^12, so no word is written and
    # every state stays at 2^16
    log("encode zeros")
    nv = 3000
    cos = np.zeros(nv, np.uint8)
    fld = np.zeros(nv * 8, np.int16)
    lo, n, freq = _tables(orc, cos, fld)
    _check(orc, cos, fld, 8192, lo, n, freq)


def test_encode_tiles_skewed_cosets(orc):
    # every vector in coset 1 but one: the coset-0 field tables hold one vector's values
    log("encode skewed cosets")
    cos, fld = _symbols(orc, 2, 16, 4096, 0.1)
    cos = np.ones_like(cos)
    cos[777] = 0
    lo, n, freq = _tables(orc, cos, fld)
    _check(orc, cos, fld, 4096, lo, n, freq)


def test_encode_tiles_symbol_outside_table(orc):
    log("encode alphabet error")
    ep = ep_mod()
    cos, fld = _symbols(orc, 2, 16, 1024, 0.3)
    lo, n, freq = _tables(orc, cos, fld)
    bad = fld.copy()
    bad[8 * 100 + 3] = int(lo[1 + 8 * int(cos[100]) + 3] + n[1 + 8 * int(cos[100]) + 3] + 5)
    st_o = orc.encode_tiles(cos, bad, 4096, 64, 12, lo, n, freq)[0]
    assert st_o != 0
    st, err, *_ = gpu_encode_tiles(cos, bad, 4096, ep.tables_struct(lo, n, freq))
    assert st == 0 and err & (1 << ERR_ALPHABET)
    badc = cos.copy()
    badc[5] = 2
    st, err, *_ = gpu_encode_tiles(badc, fld, 4096, ep.tables_struct(lo, n, freq))
    assert st == 0 and err & (1 << ERR_ALPHABET)


@pytest.mark.parametrize("F", [4096, 8192, 16384])
def test_encode_tiles_value_outside_a_byte(orc, F):
    """Tables that fit [-128, 127] let the kernel hold the fields as bytes.  A field value that
    does not fit a byte must still be an alphabet error, even where its low byte would alias a
    value of the table (257 and -255 both truncate to 1), as the oracle reports."""
    log("encode byte aliasing", F)
    ep = ep_mod()
    cos, fld = _symbols(orc, 2, 16, 2048, 0.3)
    lo, n, freq = _tables(orc, cos, fld)
    assert all(lo[t] >= -128 and lo[t] + n[t] - 1 <= 127 for t in range(1, 17) if n[t])
    for v in (257, -255, 300):
        bad = fld.copy()
        bad[8 * 700 + 2] = v
        assert orc.encode_tiles(cos, bad, F, 64, 12, lo, n, freq)[0] != 0
        st, err, *_ = gpu_encode_tiles(cos, bad, F, ep.tables_struct(lo, n, freq))
        assert st == 0 and err & (1 << ERR_ALPHABET), (v, err)


def test_encode_tiles_word_capacity(orc):
    log("encode capacity")
    ep = ep_mod()
    cos, fld = _symbols(orc, 2, 32, 2048, 0.05)
    lo, n, freq = _tables(orc, cos, fld)
    st_o, woff_o, states_o, words_o = orc.encode_tiles(cos, fld, 8192, 64, 12, lo, n, freq)
    cap = int(woff_o[-1]) - 100
    st, err, woff, mx, states, words = gpu_encode_tiles(cos, fld, 8192,
                                                        ep.tables_struct(lo, n, freq),
                                                        words_cap=cap)
    assert st == 0 and err & (1 << ERR_CAPACITY)
    assert np.array_equal(woff, woff_o)
    assert np.array_equal(words, words_o[:cap])     # nothing past the cap is written


def test_encode_tiles_argument_errors(orc):
    log("encode arguments")
    ep = ep_mod()
    cos, fld = _symbols(orc, 1, 8, 64, 0.3)
    lo, n, freq = _tables(orc, cos, fld)
    tab = ep.tables_struct(lo, n, freq)
    st, *_ = gpu_encode_tiles(cos, fld, 2048, tab)
    assert st == ERR_ARG
    st, *_ = gpu_encode_tiles(cos, fld, 4096, tab, d_fields_offset_bytes=8)
    assert st == ERR_ARG
