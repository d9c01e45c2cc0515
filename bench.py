"""Decode throughput of the lattice-rANS weight codec on one MI355X.

Workload: the 4096 x 4096 bf16 weight with log-normal row scales (sigma_r = exp(N(log 0.02,
0.5^2))), target 4.0 bits per element, 8192-field tiles -- compressed once by the library, then
decoded back to bf16 by the fused tile decoder.  One step = one ep_decompress of the whole
matrix (one kernel launch).  Eight copies of blob + output are rotated so the working set
(8 x 42 MB) exceeds the 256 MB Infinity Cache and every step reads and writes HBM.

Also timed in the same run: the E8 quantiser + histogram kernel on the same matrix (the
encoder's GPU hot path), and the CPU oracle's decode (single thread) as a baseline.
--workload selects one of the other synthetic workloads (3, 4, 5a, 5b, 1) for the same
measurement; the default line is the 4096 x 4096 one.  Workload 4 is a batch of 64 3072 x 3072
matrices: one step decodes all 64 with ep_decompress_batch (1.4 GB of output, larger than the
cache without rotation), and the line also gives one matrix's single decode.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE = 8
# rANS states per tile used for each workload unless --lanes says otherwise
DEFAULT_LANES = {}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="2",
                    help="workload key: 2 (default, the headline line), 3, 4, 5a, 5b, 1")
    ap.add_argument("--refine", type=int, default=5,
                    help="also compress with the per-row refinement (candidates; 0: skip)")
    ap.add_argument("--consumer-m", type=int, default=0,
                    help="also time the consumer product X[M x cols] @ W^T with the library "
                         "GEMM (torch.matmul) on the decoded weight, for this M (0: skip)")
    ap.add_argument("--tile-fields", type=int, default=0,
                    help="override the workload's tile size (4096, 8192 or 16384 fields). "
                         "Smaller tiles give the decoder more independent rANS states to run "
                         "at once, and cost 256 B of states per tile")
    ap.add_argument("--lanes", type=int, default=0,
                    help="rANS states per tile: 64 or 128 (two per wavefront lane); 0: the "
                         "workload's default")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="also run one traced decode (ep_decompress_traced) and report the median "
                         "clock cycles per tile of each decoder phase")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decoder shards tiles with no exchange, so a GPU's "
              "throughput is its share's; multi-GPU runs are not measured (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import entropy_coded_weight_ep_amd as ep
    import ep_synth as S

    key = int(args.workload) if args.workload.isdigit() else args.workload
    wl = S.WORKLOADS[key]
    R, C, F, target = wl["rows"], wl["cols"], wl["tile_fields"], wl["target_bpp"]
    if args.tile_fields:
        F = args.tile_fields
    K = args.lanes or DEFAULT_LANES.get(key, 64)
    dt = wl["dtype"]
    esize = S.ELEM_SIZE[dt]
    tdt = {S.BF16: torch.bfloat16, S.FP16: torch.float16, S.FP8: torch.float8_e4m3fn,
           S.INT8: torch.int8}[dt]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w_bits = S.workload_weights(key)
    t = torch.from_numpy(w_bits.view(np.uint8)).to(dev).view(tdt).view(R, C)
    n_mat = 64 if key == 4 else 1

    # compress (library: device rate search, quantiser, histogram, LS scales, tables, tile
    # encoder); the second call is the warm time
    t0 = time.time()
    comp = ep.compress(t, ep.LatticeRANSConfig(target_bpp=target, tile_fields=F, lanes=K))
    compress_s = time.time() - t0
    t0 = time.time()
    comp2 = ep.compress(t, ep.LatticeRANSConfig(target_bpp=target, tile_fields=F, lanes=K))
    compress_warm_s = time.time() - t0
    assert np.array_equal(comp.blob, comp2.blob)
    del comp2
    info = comp.info
    blob_bytes = int(comp.blob.size)
    out_bytes = R * C * esize

    # rotated copies of blob, decode tables and outputs
    blobs, tabs, outs = [], [], []
    for i in range(ROTATE):
        d = torch.from_numpy(comp.blob).to(dev)
        tb = torch.empty(ep.EP_DEC_TABLE_BYTES, dtype=torch.uint8, device=dev)
        assert ep.ep_prepare_decode(d, info, tb) == 0
        blobs.append(d)
        tabs.append(tb)
        outs.append(torch.empty((R, C), dtype=tdt, device=dev))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        k = i % ROTATE
        st = ep.ep_decompress(blobs[k], info, tabs[k], outs[k], err)
        if st:
            raise ep.EPError(st, "ep_decompress")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    assert int(err.item()) == 0, "decode reported a corrupt tile"

    # quality of the decoded tensor (relative L2 against the input, as in the design page usage)
    ref = t.float()
    rel_l2 = ((outs[(args.steps - 1) % ROTATE].float() - ref).norm() / ref.norm()).item()

    # the same matrix with the per-row rate-distortion refinement (5 resolutions per row): same
    # target, same format, so the decode above is unchanged; its error and size are reported
    refine = None
    if args.refine:
        t0 = time.time()
        rc = ep.compress(t, ep.LatticeRANSConfig(target_bpp=target, tile_fields=F,
                                                 refine=args.refine, lanes=K))
        r_s = time.time() - t0
        r_out = ep.decompress(rc)
        refine = {"candidates": args.refine, "compress_seconds": round(r_s, 3),
                  "actual_bpp": round(rc.actual_bpp, 5),
                  "rel_l2": round(((r_out.float() - ref).norm() / ref.norm()).item(), 6)}
        del r_out

    # E8 quantiser + histogram on the same matrix at the selected scale (gains from the blob's s)
    sumsq = torch.empty(R, dtype=torch.float64, device=dev)
    assert ep.ep_row_sumsq(t, dt, R, C, sumsq) == 0
    rms = torch.sqrt(sumsq / C)
    gains = torch.where(rms > 0, 1.0 / (rms * comp.scale), torch.zeros_like(rms)).float()
    cos = torch.empty(R * C // 8, dtype=torch.uint8, device=dev)
    fld = torch.empty(R * C, dtype=torch.int16, device=dev)
    hist = torch.empty(ep.HIST_BYTES // 4, dtype=torch.int32, device=dev)
    qerr = torch.zeros(1, dtype=torch.int32, device=dev)
    qsteps = max(10, args.steps // 4)
    for _ in range(3):
        ep.ep_quantize_e8(t, dt, R, C, gains, None, R, cos, fld, hist, qerr)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(qsteps):
        ep.ep_quantize_e8(t, dt, R, C, gains, None, R, cos, fld, hist, qerr)
    ev1.record()
    torch.cuda.synchronize()
    q_ms = ev0.elapsed_time(ev1) / qsteps
    q_bytes = R * C * esize + R * C // 8 + R * C * 2    # read weights, write cosets + fields

    # device tile encoder on those symbols (tables built on the device, as compress does)
    nv = R * C // 8
    d_tab = torch.empty(ep.TABLES_BYTES, dtype=torch.uint8, device=dev)
    assert ep.ep_build_tables_gpu(hist, d_tab, qerr) == 0
    h_tab = d_tab.cpu().numpy()
    ews = ep.ep_encode_workspace_bytes(nv, F)
    d_ews = torch.empty(ews, dtype=torch.uint8, device=dev)
    T = (nv + F // 8 - 1) // (F // 8)
    d_woff = torch.empty(T + 1, dtype=torch.int32, device=dev)
    d_max = torch.empty(1, dtype=torch.int32, device=dev)
    d_st = torch.empty(T * K, dtype=torch.int32, device=dev)
    d_words = torch.empty(9 * nv + 1, dtype=torch.int16, device=dev)

    def enc():
        assert ep.ep_encode_tiles_gpu(cos, fld, nv, F, h_tab, d_ews, ews, d_woff, d_max, d_st,
                                      d_words, 9 * nv + 1, qerr, lanes=K) == 0

    for _ in range(3):
        enc()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(qsteps):
        enc()
    ev1.record()
    torch.cuda.synchronize()
    e_ms = ev0.elapsed_time(ev1) / qsteps
    assert int(qerr.item()) == 0
    assert int(d_woff[-1].item()) == info.payload_words
    phases = None
    if args.phase_stamps:
        phases = phase_stamps(ep, blobs[0], info, tabs[0], outs[0], err, dev)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    # the decode against the product that consumes the weight (prefill / denoiser shapes):
    # Y[M x rows] = X[M x cols] @ W^T with the library GEMM, W being the decoded matrix
    consumer = None
    if args.consumer_m and dt in (S.BF16, S.FP16):
        Wd = outs[0].view(R, C)
        X = torch.randn(args.consumer_m, C, device=dev, dtype=torch.float32).to(tdt)
        for _ in range(3):
            torch.matmul(X, Wd.t())
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(10):
            torch.matmul(X, Wd.t())
        ev1.record()
        torch.cuda.synchronize()
        g_ms = ev0.elapsed_time(ev1) / 10
        flops = 2.0 * args.consumer_m * R * C
        consumer = {"m": args.consumer_m, "gemm_ms": round(g_ms, 4),
                    "timing": "events around the calls: at small m torch.matmul's host dispatch "
                              "can outlast its kernel, so unfused_ms is an upper bound there",
                    "gemm_tflops": round(flops / (g_ms * 1e-3) / 1e12, 1),
                    "decode_ms": round(ms, 4),
                    "decode_over_gemm": round(ms / g_ms, 4),
                    "unfused_ms": round(ms + g_ms, 4)}
        # the decode fused into the product (W never written out), on the same rotated blobs
        if args.consumer_m <= ep.EP_MM_MAX_M and C <= ep.EP_MM_MAX_COLS:
            Y = torch.empty((args.consumer_m, R), dtype=torch.float32, device=dev)

            def fused(i):
                k = i % ROTATE
                st = ep.ep_decompress_matmul(blobs[k], info, tabs[k], X, args.consumer_m, Y, err)
                if st:
                    raise ep.EPError(st, "ep_decompress_matmul")

            for i in range(3):
                fused(i)
            torch.cuda.synchronize()
            ev0.record()
            for i in range(args.steps):
                fused(i)
            ev1.record()
            torch.cuda.synchronize()
            f_ms = ev0.elapsed_time(ev1) / args.steps
            assert int(err.item()) == 0
            consumer.update({
                "fused_kernel": f"k_decode<{F // 512}, {K // 64}, {S.DTYPE_NAMES[dt]}> + MFMA "
                                "product",
                "fused_ms": round(f_ms, 4),
                "fused_vs_unfused": round((ms + g_ms) / f_ms, 4),
                "fused_over_decode": round(f_ms / ms, 4)})
            del Y
        del X

    single = None
    consumer_batch = None
    if n_mat > 1:
        # the whole batch: every matrix compressed, then one batched decode per step
        single = {"us_per_matrix_single_decode": round(ms * 1e3, 3)}
        comps = [comp]
        for m in range(1, n_mat):
            wm = S.workload_weights(key, index=m)
            tm = torch.from_numpy(wm.view(np.uint8)).to(dev).view(tdt).view(R, C)
            comps.append(ep.compress(tm, ep.LatticeRANSConfig(target_bpp=target, tile_fields=F,
                                                              lanes=K)))
            del tm
        bl = [torch.from_numpy(c.blob).to(dev) for c in comps]
        tb = []
        for c, d in zip(comps, bl):
            x = torch.empty(ep.EP_DEC_TABLE_BYTES, dtype=torch.uint8, device=dev)
            assert ep.ep_prepare_decode(d, c.info, x) == 0
            tb.append(x)
        ob = [torch.empty((R, C), dtype=tdt, device=dev) for _ in comps]
        infos = [c.info for c in comps]
        blob_bytes = sum(int(c.blob.size) for c in comps)
        out_bytes = out_bytes * n_mat
        for _ in range(args.warmup):
            assert ep.ep_decompress_batch(bl, infos, tb, ob, err) == 0
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            assert ep.ep_decompress_batch(bl, infos, tb, ob, err) == 0
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        assert int(err.item()) == 0, "batched decode reported a corrupt tile"
        single["actual_bpp_all"] = round(8.0 * blob_bytes / (n_mat * R * C), 5)
        # the same 64 matrices as 64 single launches back to back on the stream
        seq_steps = max(3, args.steps // 10)
        for _ in range(2):
            for k in range(n_mat):
                assert ep.ep_decompress(bl[k], infos[k], tb[k], ob[k], err) == 0
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(seq_steps):
            for k in range(n_mat):
                assert ep.ep_decompress(bl[k], infos[k], tb[k], ob[k], err) == 0
        ev1.record()
        torch.cuda.synchronize()
        single["us_64_single_launches"] = round(ev0.elapsed_time(ev1) / seq_steps * 1e3, 1)
        # the product that consumes each decoded matrix, fused for the whole batch
        # (ep_decompress_matmul_batch) against the batched decode plus one library GEMM each
        mc = args.consumer_m
        if mc and dt in (S.BF16, S.FP16) and mc <= ep.EP_MM_MAX_M and C <= ep.EP_MM_MAX_COLS:
            xs = [torch.randn(mc, C, device=dev, dtype=torch.float32).to(tdt)
                  for _ in range(n_mat)]
            ys = [torch.empty((mc, R), dtype=torch.float32, device=dev) for _ in range(n_mat)]

            def unfused():
                assert ep.ep_decompress_batch(bl, infos, tb, ob, err) == 0
                for k in range(n_mat):
                    torch.matmul(xs[k], ob[k].t())

            def fused_batch():
                assert ep.ep_decompress_matmul_batch(bl, infos, tb, xs, mc, ys, err) == 0

            res = {}
            for name, f in (("unfused_ms", unfused), ("fused_batch_ms", fused_batch)):
                for _ in range(2):
                    f()
                torch.cuda.synchronize()
                ev0.record()
                for _ in range(seq_steps):
                    f()
                ev1.record()
                torch.cuda.synchronize()
                res[name] = round(ev0.elapsed_time(ev1) / seq_steps, 4)
            assert int(err.item()) == 0
            consumer_batch = {
                "m": mc, "matrices": n_mat, **res,
                "fused_vs_unfused": round(res["unfused_ms"] / res["fused_batch_ms"], 4),
                "timing": "events around each form: the batched decode with one torch.matmul "
                          "per matrix, against one ep_decompress_matmul_batch call"}
            del xs, ys

    value = out_bytes / (ms * 1e-3) / 1e9
    algo_bytes = blob_bytes + out_bytes
    achieved = algo_bytes / (ms * 1e-3) / 1e9
    J = F // 512
    kname = f"k_decode<{J}, {K // 64}, {S.DTYPE_NAMES[dt]}>"
    line = {
        "metric": "decoded weight GB/s/GPU (output bytes) + % of HBM roofline; actual_bpp",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": wl["name"] + f", target {target} bpp, {F}-field tiles, {K} rANS "
                        "states per tile, one fused decode per step",
            "rows": R, "cols": C, "container": S.DTYPE_NAMES[dt], "tile_fields": F,
            "lanes": K,
            "target_bpp": target, "actual_bpp": round(info.actual_bpp, 5),
            "scale": comp.scale, "rel_l2": round(rel_l2, 6),
            "blob_bytes": blob_bytes, "output_bytes": out_bytes,
            "rotated_copies": ROTATE if n_mat == 1 else 0, "matrices": n_mat,
            "compress_seconds": round(compress_s, 3),
            "compress_seconds_warm": round(compress_warm_s, 3),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kname, str(key)),
            "kernel": kname,
            "bytes_per_launch": algo_bytes,
        },
        "quantize": {
            "kernel": f"k_quantize_e8<{S.DTYPE_NAMES[dt]}> + histogram",
            "ms": round(q_ms, 6), "bytes_per_launch": q_bytes,
            "achieved_GBs": round(q_bytes / (q_ms * 1e-3) / 1e9, 2),
            "frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "refine": refine,
        "consumer": consumer,
        "consumer_batch": consumer_batch,
        "phases": phases,
        "encode": {
            "kernel": f"k_encode_tiles<{F // 512}> + offset scan + word copy",
            "ms": round(e_ms, 6), "vectors": nv,
            "Mvectors_per_s": round(nv / (e_ms * 1e-3) / 1e6, 1),
        },
    }
    if single is not None:
        line["config"]["workload"] = wl["name"] + f", target {target} bpp, {F}-field tiles, " \
            f"{K} rANS states per tile, all {n_mat} matrices decoded by one batched call per step"
        line["config"].update(single)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(comp.blob, R * C * esize, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def decoder_source_sha() -> str:
    """Hash of the decoder's code (comments and blank space removed, so that a comment edit
    does not invalidate the counter record)."""
    import hashlib
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "entropy_coded_weight_ep_amd", "csrc")
    for f in ("ep_decode.h", "ep_device.h", "ep_internal.h"):
        src = open(os.path.join(csrc, f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy of known size), or None when no summary exists for this
    kernel and workload or the decoder sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{workload}")
    if not rec or rec.get("decoder_source_sha") != decoder_source_sha():
        return None
    return rec["traffic_bytes"]


def phase_stamps(ep, d_blob, info, d_tab, d_out, err, dev):
    """One traced decode: per tile, the shader-clock cycles of each decoder phase (median over the
    tiles)."""
    import numpy as np
    import torch

    T = int(info.tiles)
    st = torch.zeros(T * ep.EP_TRACE_STAMPS, dtype=torch.int64, device=dev)
    for _ in range(2):                                  # the second run is the one kept
        if ep.ep_decompress_traced(d_blob, info, d_tab, d_out, err, st):
            return {"error": "ep_decompress_traced refused this blob"}
    torch.cuda.synchronize()
    a = st.view(T, ep.EP_TRACE_STAMPS).cpu().numpy().astype(np.int64)
    med = lambda x: float(np.median(x))
    out = {"tiles": T, "prologue": med(a[:, 1] - a[:, 0]), "coset": med(a[:, 2] - a[:, 1])}
    prev = a[:, 2]
    for k in range(8):
        out[f"barrier{k}"] = med(a[:, 3 + 2 * k] - prev)
        out[f"phase{k}"] = med(a[:, 4 + 2 * k] - a[:, 3 + 2 * k])
        prev = a[:, 4 + 2 * k]
    out["end_check"] = med(a[:, 19] - a[:, 18])
    out["tile_total"] = med(a[:, 19] - a[:, 0])
    out["unit"] = "shader clock cycles (s_memtime; the counters of different XCDs are not aligned, "\
                  "so only differences within a tile are used)"
    return out


def cpu_baseline(blob, out_bytes, min_seconds):
    """The CPU oracle's decode of the same blob: tiles split over host threads (the oracle's C
    decode of a tile range releases the GIL), repeated for >= min_seconds; the single-thread
    rate is measured the same way and reported beside it."""
    import ctypes
    import threading

    import numpy as np

    import oracle

    oracle.build(force=False)
    info = oracle.blob_fields(blob)
    R, C, T = info["rows"], info["cols"], info["tiles"]
    out = np.zeros((R, C), oracle.bits_dtype(info["dtype"]))
    lib = oracle.lib()
    b = np.ascontiguousarray(blob)

    def run(t0, t1):
        st = lib.or_decompress(b.ctypes.data_as(ctypes.c_void_p), b.size, t0, t1,
                               out.ctypes.data_as(ctypes.c_void_p), None, None)
        assert st == 0

    def rate(threads):
        bounds = [(T * i // threads, T * (i + 1) // threads) for i in range(threads)]
        reps, t0 = 0, time.time()
        while True:
            if threads == 1:
                run(0, T)
            else:
                ws = [threading.Thread(target=run, args=bd) for bd in bounds]
                for th in ws:
                    th.start()
                for th in ws:
                    th.join()
            reps += 1
            if time.time() - t0 >= min_seconds:
                break
        el = time.time() - t0
        return out_bytes * reps / el / 1e9, reps, el

    cores = max(1, min(16, os.cpu_count() or 1))
    one, r1, e1 = rate(1)
    many, rn, en = rate(cores) if cores > 1 else (one, r1, e1)
    return {
        "value": round(many, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"whole blob decoded {rn} times in {en:.1f} s with its tiles split over "
                  f"{cores} threads; single thread: {one:.4f} GB/s ({r1} decodes in {e1:.1f} s)",
        "single_thread_value": round(one, 4),
        "cpu": cpu_model(), "host_cpus": os.cpu_count(),
    }


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty where the file does not exist)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""

if __name__ == "__main__":
    main()
