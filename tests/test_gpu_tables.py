"""The expanded decode tables (ep_prepare_decode).  Design page "EntroPack lattice compression",
*Encoding and reconstruction*: each field is rANS-coded with a table of precision 2^12, so
decoding a symbol looks up the slot x mod 2^12, which belongs to the value v with
cum(v) <= slot < cum(v) + f(v) (cum: the sum of the frequencies of the values before v).

The expected tables are that definition written out here with numpy, from the frequency records
the table offsets point at, and every slot of all 16 tables is compared bit for bit: the slot
entry f(v) | (slot - cum(v)) << 13 | (v & 127) << 25 and the value v (i16); a slot that no value
covers holds 0 in both.  The tables come from compressed blobs and from hand-made records that
reach the corners: an unused table, one value that owns every slot, a 65535-value alphabet with
scattered nonzero frequencies, long runs of zero frequencies, values far outside [-64, 63]."""

import numpy as np
import pytest

import ep_synth as S
from gpu_util import GpuBlob, dev, ep_mod, host, log

pytestmark = pytest.mark.gpu

M = 4096


def _expected(freq, lo):
    E = np.zeros(M, np.uint32)
    V = np.zeros(M, np.int16)
    cums = np.cumsum(freq, dtype=np.int64) - freq
    for i in np.flatnonzero(freq):
        f, cum = int(freq[i]), int(cums[i])
        q = np.arange(f, dtype=np.uint32)
        s = cum + q
        keep = s < M
        v = lo + int(i)
        E[s[keep]] = f | (q[keep] << 13) | (np.uint32(v & 127) << 25)
        V[s[keep]] = v
    return E, V


def _prepare(d_blob, info):
    import torch

    ep = ep_mod()
    d_tab = torch.full((ep.EP_DEC_TABLE_BYTES,), 0xAB, dtype=torch.uint8, device="cuda")
    assert ep.ep_prepare_decode(d_blob, info, d_tab) == 0
    torch.cuda.synchronize()
    t = host(d_tab)
    ent = t[:16 * M * 4].view(np.uint32).reshape(16, M)
    val = t[16 * M * 4:].view(np.int16).reshape(16, M)
    return ent, val


def _check(buf, info):
    ent, val = _prepare(dev(buf), info)
    for t in range(16):
        n = int(info.n[1 + t])
        off = int(info.table_off[1 + t])
        freq = buf[off + 8:off + 8 + 2 * n].view(np.uint16) if n else np.zeros(0, np.uint16)
        E, V = _expected(freq, int(info.lo[1 + t]))
        assert np.array_equal(ent[t], E), (t, np.flatnonzero(ent[t] != E)[:5])
        assert np.array_equal(val[t], V), (t, np.flatnonzero(val[t] != V)[:5])


@pytest.mark.parametrize("key,R,C,F", [(2, 256, 1024, None), (3, 128, 4096, 8192),
                                       ("5a", 64, 2048, None), (1, 256, 256, 4096),
                                       (4, 96, 3072, None)])
def test_tables_of_compressed_blobs(orc, key, R, C, F):
    wl = S.WORKLOADS[key]
    log("decode tables", key, R, C)
    w = S.workload_weights(key, R, C)
    st, blob, _ = orc.compress(w, wl["dtype"], wl["target_bpp"], F or wl["tile_fields"])
    assert st == 0
    gb = GpuBlob(blob)
    _check(blob, gb.info)


def _records(tables):
    """A buffer of table records (lo, n, then n u16 frequencies) and an info that points at them;
    tables[0] is the coset table, which the expansion does not read."""
    ep = ep_mod()
    info = ep.ep_blob_info()
    parts, off = [], 0
    for t, (lo, freq) in enumerate(tables):
        freq = np.asarray(freq, np.uint16)
        rec = np.concatenate([np.array([lo, freq.size], np.int32).view(np.uint8),
                              freq.view(np.uint8), np.zeros(6, np.uint8)])
        info.table_off[t] = off
        info.lo[t] = lo
        info.n[t] = freq.size
        parts.append(rec)
        off += rec.size
    return np.concatenate(parts), info


def test_tables_hand_made_corners():
    rng = np.random.default_rng(5)
    tabs = [(0, [M])]
    tabs.append((0, []))                                     # unused table
    tabs.append((-64, [M]))                                  # one value owns every slot
    tabs.append((63, [M]))
    wide = np.zeros(65535, np.uint16)                        # 4096 values of frequency 1,
    wide[np.sort(rng.choice(65535, M, replace=False))] = 1   # scattered over a 65535 alphabet
    tabs.append((-32768, wide))
    peaked = np.zeros(200, np.uint16)                        # one heavy value and zero runs
    peaked[[3, 50, 51, 199]] = [M - 3, 1, 1, 1]
    tabs.append((-100, peaked))
    for t in range(len(tabs), 17):                           # random tables with zero entries
        n = int(rng.integers(1, 3000))
        f = np.zeros(n, np.int64)
        idx = rng.choice(n, min(n, int(rng.integers(1, 400))), replace=False)
        cuts = np.sort(rng.choice(np.arange(1, M), idx.size - 1, replace=False))
        f[idx] = np.diff(np.concatenate([[0], cuts, [M]]))
        tabs.append((int(rng.integers(-2000, 100)), f))
    buf, info = _records(tabs)
    for lo, f in tabs[1:]:
        assert len(f) == 0 or int(np.sum(f)) == M
    _check(buf, info)
