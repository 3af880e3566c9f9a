#!/usr/bin/env python3
"""Benchmark: split-KV exact decode on one MI355X, 128k-token MHA workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--splits S] [--page-size P] [--tokens N]
    python bench.py --all [--steps K]

One step = one full decode over the workload's inputs, already resident in HBM,
through the public entry point tad_decode_ws (which runs the split kernel and then
the combine kernel at this size, or one fused launch on small problems); with
--page-size the K/V are first copied into a paged cache (a permuted page pool,
workloads.page_kv) and the step is tad_decode_paged_ws.  W untimed steps, then K
timed steps between two device synchronisations.  Rank 0 prints one JSON line with:

- value: KV-read throughput in GB/s (algorithmic K+V bytes / step time),
- ms_per_step and decode_step_us,
- roofline: the split kernel's algorithmic bytes per launch / its mean duration,
  from K more split launches (tad_split) each bracketed by events on the launch
  stream, against the 8 TB/s HBM peak; traffic = HBM bytes per launch measured by
  rocprofv3 counters when the committed measurement matches the current kernel
  source (else null),
- cpu_baseline: the fp64 oracle timed on this host's cores over the same workload.

--all instead prints one record per workload (1-7): the median over K steps of
tad_decode_ws, each timed with events after 512 MiB of scratch has been written
(so no K/V stays in the caches), the split kernel's median the same way, parity
against the fp64 oracle (max-abs, rel-L2, the acceptance bar), the oracle's time,
the host's CPU model and cores, the device's compute units and the seed.

Only one GPU is used: the decode of one sequence is split across the compute units
of a single device, so --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-step µs and KV-read HBM GB/s (% of peak) at 128k ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0


def kernel_source_hash(files) -> str:
    """Short sha256 over the named kernel sources (under the package's csrc/)."""
    h = hashlib.sha256()
    for f in files:
        p = os.path.join(ROOT, "long_context_attention_split_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload: int, page_size: int = 0, tokens: int = 1, scale_block: int = 0):
    """HBM bytes per split-kernel launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    tag = ("workload%d" % workload + ("_tokens%d" % tokens if tokens > 1 else "")
           + ("_block%d" % scale_block if scale_block else ""))
    if page_size:
        names = ["split_paged%d_%s_traffic.txt" % (page_size, tag)]
    else:
        names = ["split_kernel_%s_traffic.txt" % tag, "split_mfma_%s_traffic.txt" % tag]
    paths = [os.path.join(ROOT, "profiles", n) for n in names if os.path.exists(os.path.join(ROOT, "profiles", n))]
    if not paths:
        return None
    p = paths[0]
    vals = {}
    for ln in open(p):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            vals[k.strip()] = v.strip()
    files = [f.strip() for f in vals.get("kernel_sources", "").split(",") if f.strip()]
    if not files or vals.get("kernel_source_sha") != kernel_source_hash(files):
        return None
    try:
        return int(vals["fetch_bytes_per_launch"]) + int(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(c, cpu_seconds_target: float = 10.0):
    """Time the fp64 oracle over the workload's rows on this host's cores.

    The whole workload is one pass; passes repeat until about ``cpu_seconds_target``
    seconds of CPU time (wall time x threads) have been spent.  Returns the output of
    the first pass, the mean wall seconds per pass, the threads used, the rows per
    pass and the number of passes."""
    import oracle
    n_rows = c["q"].shape[0] * c["q"].shape[1]
    threads = min(len(os.sched_getaffinity(0)), n_rows)
    oracle.build(force=False)
    out, passes, total = None, 0, 0.0
    while passes == 0 or (total * threads < cpu_seconds_target and passes < 1000):
        t0 = time.perf_counter()
        o = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                              n_threads=threads, k_scale=c["k_scale"], v_scale=c["v_scale"],
                              k_scale_block=c.get("scale_block", 0), v_scale_block=c.get("scale_block", 0))
        total += time.perf_counter() - t0
        passes += 1
        if out is None:
            out = o
    return out, total / passes, threads, n_rows, passes


def copy_probe(dev, nbytes: int = 1 << 30, reps: int = 5):
    """A plain elementwise kernel over ``nbytes`` of fp32 (reads nbytes, writes nbytes):
    the known-size reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE, and a
    read+write stream rate for context."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": round(dt * 1e6, 1),
            "rw_gbs": round(2 * nbytes / dt / 1e9, 1)}


class TimingEvent:
    """A HIP event for timing only, recorded on a given stream.  Created with
    hipEventDisableSystemFence through the HIP runtime the process has loaded (torch's
    events cannot take flags): completing it then needs no system-scope cache
    writeback and invalidation, which with default events stalled the next launch on
    the stream (same steps: 311.7 us without events, 319.5 us with default ones).
    Elapsed times are read only after a device synchronisation."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            with open("/proc/self/maps") as f:
                paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
            if len(paths) != 1:
                raise RuntimeError("expected one HIP runtime in the process, found %s" % paths)
            hip = ctypes.CDLL(paths[0])
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self.h = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000)   # hipEventDisableSystemFence
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self, stream):
        rc = self._hip.hipEventRecord(self.h, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end`."""
        import ctypes
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def probe_library():
    """tad_probe_read_stream from libtad_probe.so (built beside libtad.so), or None."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_attention_split_amd",
                        "libtad_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.tad_probe_read_stream.restype = ctypes.c_int
    lib.tad_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.tad_probe_read_stream_static.restype = ctypes.c_int
    lib.tad_probe_read_stream_static.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                                 ctypes.c_void_p]
    return lib


def read_stream_probe(k, v, stream, reps: int = 10):
    """GB/s of a plain read stream over the K and V allocations, timed with events on
    `stream`, back to back; None when the probe library is missing."""
    import torch
    lib = probe_library()
    if lib is None:
        return None
    sink = torch.zeros(4096, dtype=torch.int32, device=k.device)
    bufs = []
    for t in (k, v):
        base = t if t.is_contiguous() else t.transpose(1, 2)   # [B, L, H, d] storage seen through strides
        if not base.is_contiguous():
            return None
        bufs.append((base.data_ptr(), base.numel() * base.element_size()))

    def run():
        for ptr, nbytes in bufs:
            if lib.tad_probe_read_stream(ptr, nbytes, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("read-stream probe launch failed")
    run()
    torch.cuda.synchronize()
    e0, e1 = TimingEvent(), TimingEvent()
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    total = sum(nb for _, nb in bufs) * reps
    return total / (e0.elapsed_time(e1) * 1e-3) / 1e9


def host_info():
    """CPU model and usable cores of this host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def load_inputs(args, wid, dev):
    """Workload ``wid`` on the device, with its step functions.  Returns a dict."""
    import torch
    import long_context_attention_split_amd as tad
    import workloads as W
    w = W.WORKLOADS[wid]
    t_gen = time.perf_counter()
    sb = getattr(args, "scale_block", 0)
    if sb and w.kv_dtype not in W.FP8_MAX:
        raise SystemExit("--scale-block needs an FP8 workload (6 or 7)")
    c = W.make_workload(wid, sb)
    c["scale_block"] = sb
    print("[bench] workload %d generated in %.1fs" % (wid, time.perf_counter() - t_gen), file=sys.stderr, flush=True)
    if args.tokens > 1:                    # same K/V, nq query tokens per (row, head)
        B0, Hq0, d0 = c["q"].shape
        c["q"] = W.draw_q(1000 * wid + 6, B0, Hq0 * args.tokens, d0).view(B0, Hq0, args.tokens, d0)
    nq = args.tokens
    q = c["q"].to(dev)
    table = None
    if args.page_size:
        kc, vc, table = W.page_kv(c["k"], c["v"], args.page_size, 1000 * wid, head_major=args.head_major_pages)
        k, v, table = kc.to(dev), vc.to(dev), table.to(dev)
        del kc, vc
    elif args.token_major:
        k = c["k"].transpose(1, 2).contiguous().to(dev).transpose(1, 2)
        v = c["v"].transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    else:
        k = c["k"].to(dev)
        v = c["v"].to(dev)
    sl = c["seq_lens"].to(dev) if c["seq_lens"] is not None else None
    sp = c["slopes"].to(dev) if c["slopes"] is not None else None
    ks = c["k_scale"].to(dev) if c["k_scale"] is not None else None
    vs = c["v_scale"].to(dev) if c["v_scale"] is not None else None
    B, Hq, Hkv, Lmax, d = tad.shape_of(c["q"], c["k"])
    if args.splits > 0:
        S = args.splits
    elif c["n_splits"] > 0:
        S = c["n_splits"]
    else:                                  # what tad_decode_ws picks
        S = tad.tad_auto_splits(B, Hq, Hkv, nq, Lmax, d, w.kv_dtype)
    ws = tad.workspace(q, c["k"], S)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    if sb and table is not None:           # scales cover the paged cache's logical length
        n = -(-table.shape[1] * args.page_size // sb)
        pad = lambda s: torch.cat([s, torch.ones(s.shape[0], s.shape[1], n - s.shape[2], device=dev)], 2)
        ks, vs = pad(ks), pad(vs)

    def decode():
        if table is not None:
            tad.tad_decode_paged_ws(q, k, v, table, sl, sp, S, out, ws, stream, ks, vs, sb, sb)
        else:
            tad.tad_decode_ws(q, k, v, sl, sp, S, out, ws, stream, ks, vs, sb, sb)

    def split():
        if table is not None:
            tad.tad_split_paged(q, k, v, table, sl, sp, S, ws, stream, ks, vs, sb, sb)
        else:
            tad.tad_split(q, k, v, sl, sp, S, ws, stream, ks, vs, sb, sb)

    return dict(w=w, c=c, q=q, k=k, v=v, out=out, ws=ws, S=S, nq=nq, B=B, Hq=Hq, Hkv=Hkv, Lmax=Lmax, d=d,
                stream=stream, decode=decode, split=split, kv_bytes=w.kv_bytes(c["seq_lens"]))


def time_flushed(fn, stream, reps, scratch):
    """Per-call milliseconds of fn (events on `stream`), scratch written before each call."""
    import torch
    evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
    for i in range(reps):
        if scratch is not None:
            scratch.fill_(float(i))
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def run_all(args, dev) -> int:
    """One JSON record per workload: flushed median step and split times, parity."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    cpu_model, cores = host_info()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    scratch = torch.empty(512 << 18, dtype=torch.float32, device=dev)     # 512 MiB
    oracle.build(force=False)
    for wid in sorted(W.WORKLOADS):
        x = load_inputs(args, wid, dev)
        for _ in range(args.warmup):
            x["decode"]()
        torch.cuda.synchronize()
        step_ms = time_flushed(x["decode"], x["stream"], args.steps, scratch)
        split_ms = time_flushed(x["split"], x["stream"], args.steps, scratch)
        x["decode"]()
        torch.cuda.synchronize()
        got = x["out"].cpu().double().numpy()
        c = x["c"]
        threads = min(cores, x["B"] * x["Hq"])
        t0 = time.perf_counter()
        ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                                n_threads=threads, k_scale=c["k_scale"], v_scale=c["v_scale"])
        oracle_s = time.perf_counter() - t0
        # max |V| over the valid keys, in real units, one (b, KV head) slab at a time
        vmax = 0.0
        for b in range(x["B"]):
            Lb = int(c["seq_lens"][b]) if c["seq_lens"] is not None else x["Lmax"]
            for h in range(x["Hkv"]):
                if Lb > 0:
                    a = float(c["v"][b, h, :Lb].float().abs().max())
                    vmax = max(vmax, a * (float(c["v_scale"][b, h]) if c["v_scale"] is not None else 1.0))
        tol = 1e-5 if x["w"].kv_dtype == torch.float32 else 2e-3 * vmax
        err = np.abs(got - ref)
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        us = float(np.median(step_ms)) * 1e3
        sus = float(np.median(split_ms)) * 1e3
        # the same number of bytes read by a plain stream, timed the same way (cold)
        probe = None
        plib = probe_library()
        if plib is not None:
            nbytes = int(x["kv_bytes"])
            pbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            sink = torch.zeros(4096, dtype=torch.int32, device=dev)
            stream = x["stream"]

            def read_once():
                if plib.tad_probe_read_stream(pbuf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream) != 0:
                    raise RuntimeError("read-stream probe launch failed")

            def read_static():
                if plib.tad_probe_read_stream_static(pbuf.data_ptr(), nbytes, sink.data_ptr(), cus,
                                                     stream.cuda_stream) != 0:
                    raise RuntimeError("read-stream probe launch failed")
            read_once()
            read_static()
            pus = float(np.median(time_flushed(read_once, stream, args.steps, scratch))) * 1e3
            qus = float(np.median(time_flushed(read_static, stream, args.steps, scratch))) * 1e3
            probe = {"us_median": round(pus, 2), "gbs": round(nbytes / (pus * 1e-6) / 1e9, 1),
                     "split_rate_over_probe_rate": round(pus / sus, 4),
                     "one_group_per_cu_us_median": round(qus, 2),
                     "split_rate_over_one_group_per_cu_rate": round(qus / sus, 4),
                     "what": "plain reads of the workload's K/V byte count from one contiguous buffer "
                             "(libtad_probe.so), timed like the split: 4096 four-wave work-groups handed "
                             "out by the dispatcher, and one twelve-wave work-group per CU with a fixed slice"}
            del pbuf
        rec = {
            "metric": METRIC, "record": "per-workload",
            "workload": wid, "config": {"workload": x["w"].name, "B": x["B"], "Hq": x["Hq"], "Hkv": x["Hkv"],
                                         "d": x["d"], "L": x["Lmax"], "tokens": x["nq"], "n_splits": x["S"],
                                         "kv_bytes_per_step": x["kv_bytes"]},
            "decode_step_us_median": round(us, 2),
            "decode_step_us_min": round(min(step_ms) * 1e3, 2),
            "gbs": round(x["kv_bytes"] / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100.0 * x["kv_bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "split_kernel_us_median": round(sus, 2),
            "roofline_frac_split_events": round(x["kv_bytes"] / (sus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "read_probe_cold": probe,
            "timing": "tad_decode_ws and tad_split each timed with events, median of %d calls, 512 MiB "
                      "written before each call" % args.steps,
            "parity": {"max_abs": float(err.max()), "rel_l2": rel, "tolerance_max_abs": tol,
                       "ok": bool(err.max() <= tol)},
            "oracle": {"seconds": round(oracle_s, 3), "threads": threads, "kind": "fp64 C oracle, whole workload"},
            "host": {"cpu_model": cpu_model, "cores": cores}, "device": {"compute_units": cus},
            "seed": 1000 * wid,
            "roofline_claim": wid != 1,
        }
        print(json.dumps(rec), flush=True)
        del x, got, ref, c
        torch.cuda.empty_cache()
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--all", action="store_true", help="one record per workload (1-7) instead of the bench line")
    ap.add_argument("--splits", type=int, default=0, help="chunks per head (0: automatic)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="read K/V from a paged cache with pages of this many rows (0: contiguous)")
    ap.add_argument("--head-major-pages", action="store_true",
                    help="store each page as [Hkv, page_size, d] instead of [page_size, Hkv, d]")
    ap.add_argument("--token-major", action="store_true",
                    help="contiguous K/V stored [B, L, Hkv, d] (described as [B, Hkv, L, d] by strides)")
    ap.add_argument("--tokens", type=int, default=1,
                    help="query tokens per row (several: the rows' last positions, as in "
                         "speculative decoding; K/V are read once for all of them)")
    ap.add_argument("--scale-block", type=int, default=0,
                    help="FP8 workloads: quantise K and V with one scale per block of this many keys "
                         "(a power of two, 16 to 65536) instead of one per (row, KV head)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB elementwise copy (reference for HBM byte counters)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write this many MiB of scratch between steps, outside the timed "
                         "region, so that no K/V stays in L2 or the 256 MB memory-side cache; "
                         "each step is then timed with events (default 0: steps back to back)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode splits one sequence across the compute "
              "units of a single MI355X; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import long_context_attention_split_amd as tad

    tad.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all:
        return run_all(args, dev)
    probe = copy_probe(dev) if args.copy_probe else None
    x = load_inputs(args, args.workload, dev)
    w, c, q, k, v, out, stream = x["w"], x["c"], x["q"], x["k"], x["v"], x["out"], x["stream"]
    B, Hq, Hkv, Lmax, d, S, nq, kv_bytes = x["B"], x["Hq"], x["Hkv"], x["Lmax"], x["d"], x["S"], x["nq"], x["kv_bytes"]

    # The step: tad_decode_ws (tad_decode_paged_ws), the entry point a caller uses.
    scratch = torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev) if args.flush_mib else None
    for i in range(args.warmup):
        if scratch is not None:
            scratch.fill_(-1.0 - i)
        x["decode"]()
    torch.cuda.synchronize()
    if args.flush_mib:
        ms_per_step = sum(time_flushed(x["decode"], stream, args.steps, scratch)) / args.steps
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            x["decode"]()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # The dominant kernel alone: K more split launches (tad_split), each bracketed by
    # events on the launch stream (flushed like the steps when --flush-mib is given).
    split_ms = time_flushed(x["split"], stream, args.steps, scratch)
    del scratch
    split_avg = sum(split_ms) / len(split_ms)
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    split_gbs = kv_bytes / (split_avg * 1e-3) / 1e9
    print("[bench] step %.1f us (split kernel alone %.1f us), %.0f GB/s" %
          (ms_per_step * 1e3, split_avg * 1e3, gbs), file=sys.stderr, flush=True)

    traffic = read_traffic(args.workload, args.page_size, nq, args.scale_block)
    kv_name = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float8_e4m3fn: "fp8-e4m3",
               torch.float8_e5m2: "fp8-e5m2"}[w.kv_dtype]
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "decode_step_us": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "kv_dtype": kv_name,
        "data": "synthetic",
        "config": {
            "workload": w.name + (", %d query tokens per row" % nq if nq > 1 else "")
                        + (", K/V scales per %d-key block" % args.scale_block if args.scale_block else ""),
            "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "L": Lmax, "tokens": nq,
            "n_splits": S, "kv_bytes_per_step": kv_bytes,
            "step": "tad_decode_paged_ws" if args.page_size else "tad_decode_ws",
            "timing": ("per-step events, %d MiB scratch written between steps" % args.flush_mib
                       if args.flush_mib else "steps back to back, wall clock"),
            "kv_layout": ("paged, %d-row pages%s" % (args.page_size, ", head-major" if args.head_major_pages else ""))
                         if args.page_size else ("contiguous [B, L, H, d]" if args.token_major
                                                 else "contiguous [B, H, L, d]"),
        },
        "split_kernel_us": round(split_avg * 1e3, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(split_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(split_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "split (tad_split_paged)" if args.page_size else "split (tad_split)",
            "algorithmic_bytes_per_launch": kv_bytes,
            "timing": "%d split launches after the steps, each bracketed by events on the launch stream" % args.steps,
        },
    }
    probe_gbs = read_stream_probe(k, v, stream)
    if probe_gbs:
        # a second denominator: what a plain read stream over the same K and V buffers
        # achieves on this device in this run
        result["read_probe"] = {"gbs": round(probe_gbs, 1), "frac_of_peak": round(probe_gbs / HBM_PEAK_GBS, 4),
                                "kernel": "16-byte non-temporal loads, 1 KiB per load instruction, all CUs"}
        result["roofline"]["frac_of_read_probe"] = round(split_gbs / probe_gbs, 4)

    if not args.no_cpu_baseline:
        x["decode"]()
        torch.cuda.synchronize()
        gpu_out = out.cpu().double().numpy()
        del q, k, v, x
        torch.cuda.empty_cache()
        ref, dt, threads, n_rows, passes = cpu_baseline(c)
        import numpy as np
        err = float(np.abs(gpu_out - ref).max())
        cpu_model, _ = host_info()
        result["cpu_baseline"] = {
            "value": round(kv_bytes / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": ("the whole workload (all %d (b, head) rows) per pass, fp64 C oracle, %d passes, "
                       "%.3f s wall per pass" % (n_rows, passes, dt)),
            "seconds_per_pass": round(dt, 4),
            "cpu_model": cpu_model,
        }
        result["parity_max_abs_vs_oracle"] = err
    if probe is not None:
        result["copy_probe"] = probe
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
