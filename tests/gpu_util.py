"""Helpers for the GPU tests: move numpy buffers to the device and call the C ABI of libep.so.
Nothing here computes any part of the codec."""

import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ep_mod():
    import entropy_coded_weight_ep_amd as ep

    ep.lib()
    return ep


def dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def zeros_u8(n):
    import torch

    return torch.zeros(max(int(n), 1), dtype=torch.uint8, device="cuda")


def gpu_row_sumsq(w: np.ndarray, dtype: int) -> np.ndarray:
    import torch

    ep = ep_mod()
    R, C = w.shape
    d_w = dev(w.view(np.uint8))
    out = torch.zeros(R, dtype=torch.float64, device="cuda")
    st = ep.ep_row_sumsq(d_w, dtype, R, C, out)
    assert st == 0, st
    return host(out)


def gpu_quantize(w: np.ndarray, dtype: int, gains: np.ndarray, row_sel=None, with_hist=True):
    """Returns (err word, coset, fields, hist) from ep_quantize_e8."""
    import torch

    ep = ep_mod()
    R, C = w.shape
    d_w = dev(w.view(np.uint8))
    d_g = dev(np.ascontiguousarray(gains, np.float32))
    if row_sel is not None:
        d_sel = dev(np.ascontiguousarray(row_sel, np.int64))
        nsel = len(row_sel)
    else:
        d_sel, nsel = None, R
    nv = nsel * ((C + 7) // 8)
    d_cos = torch.zeros(max(nv, 1), dtype=torch.uint8, device="cuda")
    d_fld = torch.zeros(max(nv * 8, 8), dtype=torch.int16, device="cuda")
    d_hist = torch.zeros(ep.HIST_BYTES // 4, dtype=torch.int32, device="cuda") if with_hist else None
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_quantize_e8(d_w, dtype, R, C, d_g, d_sel, nsel, d_cos, d_fld, d_hist, d_err)
    assert st == 0, st
    torch.cuda.synchronize()
    hist = host(d_hist).view(np.uint32).reshape(17, 65536) if with_hist else None
    return int(host(d_err)[0]), host(d_cos)[:nv], host(d_fld)[:nv * 8], hist


def gpu_row_lsq(w: np.ndarray, dtype: int, cos: np.ndarray, fld: np.ndarray):
    import torch

    ep = ep_mod()
    R, C = w.shape
    num = torch.zeros(R, dtype=torch.float64, device="cuda")
    den4 = torch.zeros(R, dtype=torch.int64, device="cuda")
    st = ep.ep_row_lsq(dev(w.view(np.uint8)), dtype, R, C, dev(cos), dev(fld), num, den4)
    assert st == 0, st
    return host(num), host(den4)


class GpuBlob:
    """A blob on the device with its decode tables prepared."""

    def __init__(self, blob: np.ndarray):
        import torch

        ep = ep_mod()
        self.blob = blob
        st, self.info = ep.ep_blob_parse(blob)
        assert st == 0, st
        self.d_blob = dev(blob)
        self.d_tab = torch.zeros(ep.EP_DEC_TABLE_BYTES, dtype=torch.uint8, device="cuda")
        assert ep.ep_prepare_decode(self.d_blob, self.info, self.d_tab) == 0

    def pitch(self):
        return (self.info.cols + 7) // 8 * 8

    def out_bytes(self):
        esize = {1: 2, 2: 2, 3: 1, 4: 1, 5: 4}[self.info.dtype]
        return self.info.rows * self.pitch() * esize

    def decode(self, d_out=None, flags=None):
        """Returns (err word, output container bits as numpy [rows, cols]).  flags: None for
        ep_decompress, else the ep_decompress_ex layout flags."""
        import torch

        ep = ep_mod()
        if d_out is None:
            d_out = torch.zeros(self.out_bytes(), dtype=torch.uint8, device="cuda")
        d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if flags is None:
            st = ep.ep_decompress(self.d_blob, self.info, self.d_tab, d_out, d_err)
        else:
            st = ep.ep_decompress_ex(self.d_blob, self.info, self.d_tab, d_out, d_err, flags)
        assert st == 0, st
        torch.cuda.synchronize()
        out = host(d_out)
        dt = self.info.dtype
        npdt = {1: np.uint16, 2: np.uint16, 3: np.uint8, 4: np.int8, 5: np.uint32}[dt]
        full = out.view(npdt).reshape(self.info.rows, self.pitch())
        return int(host(d_err)[0]), np.ascontiguousarray(full[:, :self.info.cols])


def gpu_compress(w: np.ndarray, dtype: int, target_bpp: float, tile_fields: int,
                 force_scale: float = 0.0, refine: int = 0, lanes: int = 64,
                 sample_rows: int = 256, search_iters: int = 40, rate_check: bool = True):
    """Library compress of a device copy of w -> (blob bytes, s)."""
    import torch

    ep = ep_mod()
    tmap = {1: torch.bfloat16, 2: torch.float16, 3: torch.float8_e4m3fn, 4: torch.int8,
            5: torch.float32}
    t = dev(w.view(np.uint8)).view(tmap[dtype]).view(w.shape)
    cfg = ep.LatticeRANSConfig(target_bpp=target_bpp, tile_fields=tile_fields,
                               force_scale=force_scale, refine=refine, lanes=lanes,
                               sample_rows=sample_rows, search_iters=search_iters,
                               rate_check=rate_check)
    c = ep.compress(t, cfg)
    return c.blob, c.scale


def gpu_encode_tiles(cos: np.ndarray, fld: np.ndarray, tile_fields: int, tables: np.ndarray,
                     words_cap=None, d_fields_offset_bytes: int = 0, lanes: int = 64):
    """ep_encode_tiles_gpu on device copies of the symbols -> (status, err word, word_off,
    max_tile_words, states, words[:min(word_off[-1], cap)]).  tables: ep_tables byte layout."""
    import torch

    ep = ep_mod()
    nv = int(cos.size)
    V = tile_fields // 8
    T = (nv + V - 1) // V
    cap = 9 * nv + 1 if words_cap is None else int(words_cap)
    d_cos = dev(np.ascontiguousarray(cos, np.uint8))
    raw = np.zeros(nv * 16 + 64, np.uint8)
    d_raw = dev(raw)
    d_fld = d_raw[d_fields_offset_bytes:d_fields_offset_bytes + nv * 16]
    d_fld.copy_(dev(np.ascontiguousarray(fld, np.int16).view(np.uint8)))
    wsb = ep.ep_encode_workspace_bytes(nv, tile_fields)
    d_ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    d_woff = torch.full((T + 1,), -1, dtype=torch.int32, device="cuda")
    d_max = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_states = torch.zeros(max(T, 1) * lanes, dtype=torch.int32, device="cuda")
    d_words = torch.zeros(max(cap, 1), dtype=torch.int16, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = ep.ep_encode_tiles_gpu(d_cos, d_fld, nv, tile_fields, tables, d_ws, wsb, d_woff, d_max,
                                d_states, d_words, cap, d_err, lanes=lanes)
    torch.cuda.synchronize()
    woff = host(d_woff).view(np.uint32)
    n = min(int(woff[-1]), cap) if st == 0 else 0
    return (st, int(host(d_err)[0]), woff, int(host(d_max).view(np.uint32)[0]),
            host(d_states).view(np.uint32), host(d_words).view(np.uint16)[:n])
