"""ctypes wrapper around the C oracle (oracle/ep_oracle.c).

TEST INFRASTRUCTURE ONLY: the oracle is the plain CPU statement of what the lattice-rANS codec
computes.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package; the HIP library never links, loads or calls it.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB = os.path.join(HERE, "_build", "libep_oracle.so")

OK, ERR_ARG, ERR_SHAPE, ERR_DTYPE, ERR_NONFINITE, ERR_RANGE, ERR_ALPHABET, ERR_CORRUPT, \
    ERR_VERSION = range(9)
ERR_CAPACITY = 10
NTABLES, NBINS = 17, 65536


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, IEEE semantics)."""
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        L = C.CDLL(LIB)
        P = C.c_void_p
        i64, i32, dbl = C.c_int64, C.c_int, C.c_double
        sig = {
            "or_widen": (C.c_float, [i32, C.c_uint32]),
            "or_narrow": (C.c_uint32, [i32, C.c_float]),
            "or_widen_array": (None, [i32, P, i64, P]),
            "or_narrow_array": (None, [i32, P, i64, P]),
            "or_row_sumsq": (None, [i32, P, i64, i64, P]),
            "or_gain": (C.c_float, [dbl, i64, dbl]),
            "or_e8_nearest": (i32, [P, P]),
            "or_e8_brute": (i32, [P, P, P]),
            "or_e8_certificate": (i64, [P, i64, dbl, P]),
            "or_e8_vs_brute": (i64, [P, i64, dbl]),
            "or_e8_mse": (dbl, [P, i64]),
            "or_fields_from_point": (None, [i32, P, P]),
            "or_point_from_fields": (None, [P, P]),
            "or_field_bijection_box": (i64, [i32]),
            "or_quantize": (i32, [i32, P, i64, i64, P, P, i64, P, P]),
            "or_histogram": (None, [P, P, i64, P]),
            "or_normalize": (i32, [P, C.c_int32, i32, P]),
            "or_build_tables": (i32, [P, i32, P, P, P]),
            "or_build_tables_ex": (i32, [P, i32, i32, P, P, P]),
            "or_escape_keep": (None, [P, i32, P]),
            "or_substitute": (i32, [i32, C.c_uint32, P]),
            "or_exceptions": (i64, [P, P, i64, P, P, P, P, P]),
            "or_blob_exceptions": (i32, [P, i64, P]),
            "or_row_lsq": (None, [i32, P, i64, i64, P, P, P, P]),
            "or_alpha": (C.c_float, [dbl, i64]),
            "or_encode_tiles": (i32, [P, P, i64, i32, i32, i32, P, P, P, P, P, P, i64]),
            "or_decode_tiles": (i32, [P, P, P, i64, i32, i32, i32, P, P, P, i64, i64, P, P]),
            "or_compress": (i32, [i32, P, i64, i64, dbl, i32, dbl, i32, P, i64, P, P]),
            "or_rate_costs": (None, [P]),
            "or_row_rates": (None, [P, P, i64, i64, P, P, P, P, P]),
            "or_refine_select": (dbl, [P, P, i64, i32, i64, P]),
            "or_compress_bound": (i32, [i64, i64, i32, P]),
            "or_decompress": (i32, [P, i64, i64, i64, P, P, P]),
            "or_blob_fields": (i32, [P, i64, P, P, P, P, P, P, P, P]),
            "or_estimate_bpp": (dbl, [i32, P, i64, i64, P, i32, dbl]),
            "or_search_scale": (dbl, [i32, P, i64, i64, P, i32, dbl]),
            "or_estimate_bpp_ex": (dbl, [i32, P, i64, i64, P, i32, i32, i32, dbl]),
            "or_search_scale_ex": (dbl, [i32, P, i64, i64, P, i32, i32, i32, i32, dbl]),
            "or_compress_cfg": (i32, [i32, P, i64, i64, P, P, i64, P, P]),
            "or_check_scale": (dbl, [i32, P, i64, i64, P, i32, i32, dbl, dbl]),
            "or_config_default": (None, [P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


# ----------------------------------------------------------------------------------------------
# numpy-level helpers
# ----------------------------------------------------------------------------------------------
def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits)
    out = np.empty(bits.size, np.float32)
    lib().or_widen_array(dtype, _p(bits), bits.size, _p(out))
    return out.reshape(bits.shape)


def bits_dtype(dtype: int):
    """numpy type of a container's raw bits."""
    return {1: np.uint16, 2: np.uint16, 3: np.uint8, 4: np.int8, 5: np.uint32}[dtype]


def narrow(values: np.ndarray, dtype: int) -> np.ndarray:
    v = np.ascontiguousarray(values, np.float32)
    out = np.empty(v.size, bits_dtype(dtype))
    lib().or_narrow_array(dtype, _p(v), v.size, _p(out))
    return out.reshape(v.shape)


def row_sumsq(w: np.ndarray, dtype: int) -> np.ndarray:
    w = np.ascontiguousarray(w)
    out = np.empty(w.shape[0], np.float64)
    lib().or_row_sumsq(dtype, _p(w), w.shape[0], w.shape[1], _p(out))
    return out


def gains(sumsq: np.ndarray, cols: int, s: float) -> np.ndarray:
    return np.array([lib().or_gain(float(v), cols, s) for v in sumsq], np.float32)


def e8_nearest(x: np.ndarray):
    """x: (..., 8) float32 -> (coset uint8 [...], z int32 [..., 8])."""
    xs = np.ascontiguousarray(x, np.float32).reshape(-1, 8)
    cos = np.empty(xs.shape[0], np.uint8)
    z = np.empty((xs.shape[0], 8), np.int32)
    L = lib()
    for i in range(xs.shape[0]):
        zi = np.empty(8, np.int32)
        cos[i] = L.or_e8_nearest(_p(xs[i]), _p(zi))
        z[i] = zi
    return cos.reshape(x.shape[:-1]), z.reshape(x.shape)


def e8_brute(x: np.ndarray):
    xi = np.ascontiguousarray(x, np.float32).reshape(8)
    z = np.empty(8, np.int32)
    d = C.c_longdouble()
    c = lib().or_e8_brute(_p(xi), _p(z), C.byref(d))
    return c, z, float(d.value)


def fields_from_point(coset: int, z) -> np.ndarray:
    zi = np.ascontiguousarray(z, np.int32)
    f = np.empty(8, np.int32)
    lib().or_fields_from_point(int(coset), _p(zi), _p(f))
    return f


def point_from_fields(f) -> np.ndarray:
    fi = np.ascontiguousarray(f, np.int32)
    z = np.empty(8, np.int32)
    lib().or_point_from_fields(_p(fi), _p(z))
    return z


def quantize(w: np.ndarray, dtype: int, gains_: np.ndarray, row_sel=None):
    w = np.ascontiguousarray(w)
    R, Cc = w.shape
    g = np.ascontiguousarray(gains_, np.float32)
    if row_sel is not None:
        sel = np.ascontiguousarray(row_sel, np.int64)
        nsel = sel.size
        sel_p = _p(sel)
    else:
        nsel, sel_p = R, None
    nv = nsel * ((Cc + 7) // 8)
    cos = np.empty(nv, np.uint8)
    fld = np.empty(nv * 8, np.int16)
    st = lib().or_quantize(dtype, _p(w), R, Cc, _p(g), sel_p, nsel, _p(cos), _p(fld))
    return st, cos, fld


def histogram(cos: np.ndarray, fld: np.ndarray) -> np.ndarray:
    counts = np.empty((NTABLES, NBINS), np.uint64)
    lib().or_histogram(_p(np.ascontiguousarray(cos)), _p(np.ascontiguousarray(fld)), cos.size,
                       _p(counts))
    return counts


def normalize(counts, precision: int = 12):
    c = np.ascontiguousarray(counts, np.uint64)
    f = np.empty(c.size, np.uint16)
    st = lib().or_normalize(_p(c), c.size, precision, _p(f))
    return st, f


def build_tables(counts: np.ndarray, precision: int = 12):
    lo = np.empty(NTABLES, np.int32)
    n = np.empty(NTABLES, np.uint32)
    freq = np.zeros((NTABLES, NBINS), np.uint16)
    st = lib().or_build_tables(_p(np.ascontiguousarray(counts, np.uint64)), precision, _p(lo),
                               _p(n), _p(freq))
    return st, lo, n, freq


def build_tables_escapes(counts: np.ndarray, precision: int = 12):
    """Tables with escapes allowed: a field table with more than 2^P distinct values keeps the
    2^P most frequent ones."""
    lo = np.empty(NTABLES, np.int32)
    n = np.empty(NTABLES, np.uint32)
    freq = np.zeros((NTABLES, NBINS), np.uint16)
    st = lib().or_build_tables_ex(_p(np.ascontiguousarray(counts, np.uint64)), precision, 1,
                                  _p(lo), _p(n), _p(freq))
    return st, lo, n, freq


def escape_keep(counts_one_table: np.ndarray, precision: int = 12) -> np.ndarray:
    kept = np.zeros(NBINS, np.uint8)
    lib().or_escape_keep(_p(np.ascontiguousarray(counts_one_table, np.uint64)), precision,
                         _p(kept))
    return kept.astype(bool)


def substitute(lo: int, n: int, freq_one_table: np.ndarray) -> int:
    return lib().or_substitute(int(lo), int(n), _p(np.ascontiguousarray(freq_one_table, np.uint16)))


def exceptions(cos, fld, lo, n, freq):
    """(idx = v | coset << 31, true fields [X, 8]) of the vectors with an escaped field."""
    cos = np.ascontiguousarray(cos, np.uint8)
    fld = np.ascontiguousarray(fld, np.int16)
    lo = np.ascontiguousarray(lo, np.int32)
    n = np.ascontiguousarray(n, np.uint32)
    freq = np.ascontiguousarray(freq, np.uint16)
    m = lib().or_exceptions(_p(cos), _p(fld), cos.size, _p(lo), _p(n), _p(freq), None, None)
    idx = np.zeros(max(m, 1), np.uint32)
    xf = np.zeros((max(m, 1), 8), np.int16)
    lib().or_exceptions(_p(cos), _p(fld), cos.size, _p(lo), _p(n), _p(freq), _p(idx), _p(xf))
    return idx[:m], xf[:m]


def blob_exceptions(blob: np.ndarray) -> int:
    m = C.c_int64()
    st = lib().or_blob_exceptions(_p(blob), blob.size, C.byref(m))
    if st:
        raise ValueError(f"oracle blob parse failed: {st}")
    return m.value


def row_lsq(w: np.ndarray, dtype: int, cos: np.ndarray, fld: np.ndarray):
    w = np.ascontiguousarray(w)
    R, Cc = w.shape
    num = np.empty(R, np.float64)
    den4 = np.empty(R, np.int64)
    lib().or_row_lsq(dtype, _p(w), R, Cc, _p(cos), _p(fld), _p(num), _p(den4))
    return num, den4


def alpha(num: float, den4: int) -> float:
    return lib().or_alpha(float(num), int(den4))


def encode_tiles(cos, fld, tile_fields, lanes, precision, lo, n, freq):
    nv = cos.size
    V = tile_fields // 8
    T = (nv + V - 1) // V
    woff = np.empty(T + 1, np.uint32)
    states = np.empty(T * lanes, np.uint32)
    cap = 9 * nv + 1
    words = np.empty(cap, np.uint16)
    st = lib().or_encode_tiles(_p(cos), _p(fld), nv, tile_fields, lanes, precision, _p(lo), _p(n),
                               _p(freq), _p(woff), _p(states), _p(words), cap)
    return st, woff, states, words[: int(woff[-1])] if st == 0 else words


def decode_tiles(woff, states, words, nv, tile_fields, lanes, precision, lo, n, freq, t0=0,
                 t1=None):
    V = tile_fields // 8
    T = (nv + V - 1) // V
    t1 = T if t1 is None else t1
    cos = np.zeros(nv, np.uint8)
    fld = np.zeros(nv * 8, np.int16)
    words = np.ascontiguousarray(words, np.uint16)
    if words.size == 0:
        words = np.zeros(1, np.uint16)
    st = lib().or_decode_tiles(_p(woff), _p(states), _p(words), nv, tile_fields, lanes, precision,
                               _p(lo), _p(n), _p(freq), t0, t1, _p(cos), _p(fld))
    return st, cos, fld


class OrConfig(C.Structure):
    """or_config: the oracle's compression settings."""
    _fields_ = [("target_bpp", C.c_double), ("tile_fields", C.c_int), ("lanes", C.c_int),
                ("sample_rows", C.c_int), ("search_iters", C.c_int), ("refine", C.c_int),
                ("force_scale", C.c_double), ("rate_check", C.c_int)]


def compress(w: np.ndarray, dtype: int, target_bpp: float, tile_fields: int,
             force_s: float = 0.0, refine: int = 0, lanes: int = 64, sample_rows: int = 256,
             search_iters: int = 40, rate_check: int = 1):
    """Returns (status, blob bytes as uint8 array, s).  refine: 0, or the odd number (<= 9) of
    candidate resolutions per row of the rate-distortion refinement; lanes: rANS states per
    tile (64 or 128); sample_rows / search_iters: the rate search's sample and bisection steps."""
    w = np.ascontiguousarray(w)
    R, Cc = w.shape
    bound = C.c_int64()
    st = lib().or_compress_bound(R, Cc, tile_fields, C.byref(bound))
    if st:
        return st, None, 0.0
    blob = np.empty(bound.value, np.uint8)
    nbytes = C.c_int64()
    s = C.c_double()
    cfg = OrConfig(float(target_bpp), int(tile_fields), int(lanes), int(sample_rows),
                   int(search_iters), int(refine), float(force_s), int(rate_check))
    st = lib().or_compress_cfg(dtype, _p(w), R, Cc, C.byref(cfg), _p(blob), blob.size,
                               C.byref(nbytes), C.byref(s))
    if st:
        return st, None, s.value
    return st, blob[: nbytes.value].copy(), s.value


def blob_fields(blob: np.ndarray) -> dict:
    r, c, dt, F, T, s, W, tb = (C.c_int64(), C.c_int64(), C.c_int(), C.c_int(), C.c_int64(),
                                C.c_double(), C.c_int64(), C.c_int64())
    st = lib().or_blob_fields(_p(blob), blob.size, C.byref(r), C.byref(c), C.byref(dt),
                              C.byref(F), C.byref(T), C.byref(s), C.byref(W), C.byref(tb))
    if st:
        raise ValueError(f"oracle blob parse failed: {st}")
    return dict(rows=r.value, cols=c.value, dtype=dt.value, tile_fields=F.value, tiles=T.value,
                s=s.value, payload_words=W.value, table_bytes=tb.value)


def decompress(blob: np.ndarray, t0: int = 0, t1: int = -1, want_fields: bool = False):
    """Returns (status, out container bits [R, C], coset, fields)."""
    info = blob_fields(blob)
    R, Cc, dt = info["rows"], info["cols"], info["dtype"]
    out = np.zeros((R, Cc), bits_dtype(dt))
    nv = R * ((Cc + 7) // 8)
    cos = np.zeros(nv, np.uint8) if want_fields else None
    fld = np.zeros(nv * 8, np.int16) if want_fields else None
    st = lib().or_decompress(_p(blob), blob.size, t0, t1, _p(out),
                             _p(cos) if want_fields else None, _p(fld) if want_fields else None)
    return st, out, cos, fld


def decompress_matmul(blob: np.ndarray, x_bits: np.ndarray):
    """The decoded tensor inside a product (EntroPack abstract: decoding during inference, for
    workloads such as Transformer prefill and diffusion denoising), by its plain definition:
    Y[i][n] = sum_k X[i][k] W[n][k], with W the blob's decode (its container values) and X the
    container values x_bits [m, cols] of the same container, formed in fp64 by a library product.
    Returns (status, Y [m, rows] fp64, B [m, rows] = sum_k |X[i][k]| |W[n][k]|): B sizes the
    rounding error of any fp32 evaluation of the same sums."""
    st, wb, _, _ = decompress(blob)
    dt = blob_fields(blob)["dtype"]
    W = widen(wb, dt).astype(np.float64)
    X = widen(np.ascontiguousarray(x_bits), dt).astype(np.float64)
    return st, X @ W.T, np.abs(X) @ np.abs(W).T


def estimate_bpp(w, dtype, tile_fields, s, sumsq=None, lanes: int = 64, sample_rows: int = 256):
    w = np.ascontiguousarray(w)
    ss = row_sumsq(w, dtype) if sumsq is None else sumsq
    return lib().or_estimate_bpp_ex(dtype, _p(w), w.shape[0], w.shape[1], _p(ss), tile_fields,
                                    int(lanes), int(sample_rows), s)


def search_scale(w, dtype, tile_fields, target_bpp, sumsq=None, lanes: int = 64,
                 sample_rows: int = 256, search_iters: int = 40):
    w = np.ascontiguousarray(w)
    ss = row_sumsq(w, dtype) if sumsq is None else sumsq
    return lib().or_search_scale_ex(dtype, _p(w), w.shape[0], w.shape[1], _p(ss), tile_fields,
                                    int(lanes), int(sample_rows), int(search_iters), target_bpp)


def check_scale(w, dtype, tile_fields, target_bpp, s0, sumsq=None, lanes: int = 64):
    w = np.ascontiguousarray(w)
    ss = row_sumsq(w, dtype) if sumsq is None else sumsq
    return lib().or_check_scale(dtype, _p(w), w.shape[0], w.shape[1], _p(ss), tile_fields,
                                int(lanes), float(target_bpp), float(s0))


def rate_costs() -> np.ndarray:
    """Fixed-point code lengths (2^-16 bit) of frequencies 1..2^P; entry 0: a value absent from
    the model."""
    c = np.empty((1 << 12) + 1, np.uint32)
    lib().or_rate_costs(_p(c))
    return c


def row_rates(cos, fld, rows, cols, lo, n, freq, cost) -> np.ndarray:
    out = np.empty(rows, np.int64)
    lib().or_row_rates(_p(np.ascontiguousarray(cos, np.uint8)),
                       _p(np.ascontiguousarray(fld, np.int16)), rows, cols,
                       _p(np.ascontiguousarray(lo, np.int32)),
                       _p(np.ascontiguousarray(n, np.uint32)),
                       _p(np.ascontiguousarray(freq, np.uint16)),
                       _p(np.ascontiguousarray(cost, np.uint32)), _p(out))
    return out


def refine_select(D: np.ndarray, Rq: np.ndarray, budget_q: int):
    """Lagrangian selection over candidates: D, Rq are [rows, nc].  Returns (lambda, sel)."""
    D = np.ascontiguousarray(D, np.float64)
    Rq = np.ascontiguousarray(Rq, np.int64)
    rows, nc = D.shape
    sel = np.empty(rows, np.int32)
    lam = lib().or_refine_select(_p(D), _p(Rq), rows, nc, int(budget_q), _p(sel))
    return lam, sel
