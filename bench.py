#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * prefill  fa_fwd    B1 H32 N4096 d128, causal, bf16 (1 % of key rows ×8)
  * decode   fa_decode B16 H32 Lkv32768 d128, 64 KV splits, bf16
W untimed warm-up steps, then K timed steps between device synchronisations.
Each call is also timed with HIP events recorded on the stream it runs on
(torch's current stream), created with hipEventDisableSystemFence so that
recording them adds no cache writeback or invalidation between the calls;
they give the per-kernel figures:
  * value            prefill TFLOP/s = 4·N²·d·B·H / 2 (causal) ÷ fa_fwd time
  * decode.value     GB/s of algorithmic bytes (K, V once; q in; O, LSE out)
  * roofline         fa_fwd against the bf16 dense MFMA peak (2.5166 PFLOP/s)
  * roofline_decode  the decode pair against the HBM peak (8 TB/s)
  * decode_gqa       grouped-query decode (B16, 32 query heads over 8 K/V heads,
                     Lkv 32768, d128), timed on its own after the step
  * block_sparse     fa_fwd_block_sparse on B1 H16 N16384 d128 with a seeded
                     block mask (own and first key block, 10 % of the rest),
                     against fa_fwd on the same inputs: TFLOP/s of the kept
                     blocks and the speed-up over the dense call
  * decode_paged     the same grouped-query decode over the cache laid out in
                     64-key pages in a seeded random order (fa_decode_paged)
  * backward         fa_bwd on the prefill workload (the step's O and L, a
                     seeded dO), timed on its own after the step: TFLOP/s of
                     the five N×N×d products, 10·N²·d·B·H / 2 (causal)
  * prefill_workloads  fa_fwd on each prefill workload (B1 H1 N256 d64; B8 H12
                     N1024 d64 causal; the Llama-3-shaped one; B1 H16 N16384 d128),
                     timed warm (back to back) and cold (caches flushed between calls)
  * device           name, architecture, ROCm and HIP versions, and the gfx clock
                     amd-smi reports while the prefill runs
  * cpu_baseline     the fp64 oracle on a bounded sample of the same workload,
                     on this host's cores (rank 0, N=1 only)
Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 256 * 4 * 1024 * 2.4e9 / 1e12   # 2516.6: 256 CUs × 4 SIMDs × 1024 FLOP/clk × 2.4 GHz
HBM_PEAK_GBS = 8000.0

METRIC = "fwd attention TFLOP/s & % bf16 MFMA peak; split-KV decode HBM GB/s & % peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "fwd", "decode", "gqa", "bwd", "sparse", "fp8", "copy", "workloads"],
                    default="all",
                    help="time one call kind only (for counter collection); 'gqa' is the grouped-query "
                         "decode and 'bwd' the backward, both measured after the step; 'copy' times a "
                         "plain 1 GiB device-to-device copy, the reference for scaling HBM byte counters")
    ap.add_argument("--prefill", default=None, metavar="WORKLOAD",
                    help="with --only fwd: time the forward on this synth workload instead (counter runs "
                         "of other shapes, e.g. gpt2_small_causal_b8h12n1024d64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd-atomic", action="store_true",
                    help="skip the fa_bwd_atomic comparison in the backward leg (counter runs of fa_bwd alone)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the oracle sample")
    ap.add_argument("--events", choices=["nofence", "torch"], default="nofence",
                    help="timing events: HIP events created with hipEventDisableSystemFence (default; recording "
                         "one writes back and invalidates no cache), or torch.cuda.Event (a system-scope fence "
                         "at each record)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 --pmc (JSON), if present")
    ap.add_argument("--make-traffic", metavar="DIR",
                    help="write --traffic from rocprofv3 --pmc csv output under DIR/<COUNTER>_<kind>/ "
                         "(COUNTER in FETCH_SIZE, WRITE_SIZE; kind in fwd, decode, gqa, bwd, sparse, copy) and exit")
    return ap.parse_args()


class HipTimingEvent:
    """A HIP event used only to time work on torch's current stream, created with
    hipEventDisableSystemFence: recording it performs no system-scope fence, so it
    neither writes back and invalidates the caches nor delays the next kernel (which
    a default event does at every record).  Same interface as torch.cuda.Event."""
    _hip = None

    @classmethod
    def runtime(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:  # the HIP runtime torch (and libfa.so) already use
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            hip = ctypes.CDLL(path or "libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        import torch
        self._torch, self._ctypes, self._hip = torch, ctypes, self.runtime()
        self.ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000)  # hipEventDisableSystemFence
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = self._hip.hipEventRecord(self.ev, self._ctypes.c_void_p(self._torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = self._ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(self._ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        hip = getattr(self, "_hip", None)
        if hip is not None and self.ev:
            try:
                hip.hipEventDestroy(self.ev)
            except Exception:  # interpreter shutdown
                pass


EVENT_KIND = "nofence"


def Event():
    """A timing event of the kind --events selects."""
    if EVENT_KIND == "torch":
        import torch
        return torch.cuda.Event(enable_timing=True)
    return HipTimingEvent()


# Kernels whose HBM bytes are reported, and the sources each one is built from: a traffic
# figure taken from an older build of those sources is stale and reported as null.
TRAFFIC_KERNELS = {
    "fwd": (["fa_fwd_kernel"], ["fa_fwd.hip", "fa_device.h", "fa_internal.h"]),
    "decode": (["fa_decode_split_kernel", "fa_decode_combine_kernel"], ["fa_decode.hip", "fa_internal.h"]),
    "gqa": (["fa_decode_split_kernel", "fa_decode_combine_kernel"], ["fa_decode.hip", "fa_internal.h"]),
    "bwd": (["fa_bwd_dq_kernel", "fa_bwd_dkdv_pair_kernel"],
            ["fa_bwd.hip", "fa_device.h", "fa_internal.h"]),
    "sparse": (["fa_fwd_kernel<128, false, true>"], ["fa_fwd.hip", "fa_device.h", "fa_internal.h"]),
    "copy": (["copyBuffer"], []),
}


def sources_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_attention_31_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_means(folder, counter):
    """Mean per-dispatch value of ``counter`` for each kernel name in a rocprofv3 csv run."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                sums[name] = sums.get(name, 0.0) + float(row["Counter_Value"])
                counts[name] = counts.get(name, 0) + 1
    return {n: sums[n] / counts[n] for n in sums}


def make_traffic(args):
    """HBM bytes per launch = FETCH_SIZE·f_r + WRITE_SIZE·f_w (KiB), where f_r and f_w make the
    counters of a plain 1 GiB copy read exactly 1 GiB and write exactly 1 GiB."""
    def per_launch(kind, counter):
        means = counter_means(os.path.join(args.make_traffic, f"{counter}_{kind}"), counter)
        total = 0.0
        for pat in TRAFFIC_KERNELS[kind][0]:
            hits = [v for n, v in means.items() if pat in n]
            if not hits:
                raise SystemExit(f"no {counter} rows for {pat} under {args.make_traffic}")
            total += max(hits)
        return total

    gib_kib = float(1 << 20)
    f_r = gib_kib / per_launch("copy", "FETCH_SIZE")
    f_w = gib_kib / per_launch("copy", "WRITE_SIZE")
    out = {"method": "rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), scaled by a 1 GiB copy",
           "fetch_scale": round(f_r, 4), "write_scale": round(f_w, 4)}
    for kind in ("fwd", "decode", "gqa", "bwd", "sparse"):
        if not os.path.isdir(os.path.join(args.make_traffic, f"FETCH_SIZE_{kind}")):
            continue
        fk, wk = per_launch(kind, "FETCH_SIZE"), per_launch(kind, "WRITE_SIZE")
        out[kind] = {"bytes_per_launch": round((fk * f_r + wk * f_w) * 1024.0),
                     "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                     "kernels": TRAFFIC_KERNELS[kind][0],
                     "sources_sha256": sources_digest(TRAFFIC_KERNELS[kind][1])}
    with open(args.traffic, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))
    return 0


def traffic_bytes(traffic, kind):
    """Measured HBM bytes per launch, or None when absent or taken from other kernel sources."""
    ent = traffic.get(kind)
    if not isinstance(ent, dict) or ent.get("sources_sha256") != sources_digest(TRAFFIC_KERNELS[kind][1]):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(wf, wd, q, k, v, qd, kd, vd, budget_s):
    """Time the oracle (as it is) on a bounded sample: whole heads of each workload, prefill
    first (at most half the budget), then decode heads until the budget is spent."""
    threads = min(len(os.sched_getaffinity(0)), 16)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, str(threads))
    from oracle import attention_ref, decode_ref
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(threads)
        used = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        used = threads
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    heads = 0
    while heads < wf.H and time.perf_counter() - t0 < budget_s * 0.5:
        attention_ref(qc[:, heads:heads + 1], kc[:, heads:heads + 1], vc[:, heads:heads + 1], wf.scale, wf.causal)
        heads += 1
    t_f = time.perf_counter() - t0
    flops = 4.0 * wf.N * wf.N * wf.d * heads / (2 if wf.causal else 1)
    t1 = time.perf_counter()
    dheads = 0
    while dheads < wd.B * wd.H and time.perf_counter() - t0 < budget_s:
        b, h = divmod(dheads, wd.H)
        decode_ref(qd[b:b + 1, h:h + 1].cpu(), kd[b:b + 1, h:h + 1].cpu(), vd[b:b + 1, h:h + 1].cpu(), wd.scale)
        dheads += 1
    t_d = time.perf_counter() - t1
    dbytes = dheads * (2 * wd.lkv * wd.d * 2 + 2 * wd.d * 2 + 4)
    return {
        "value": flops / t_f / 1e12,
        "unit": "TFLOP/s",
        "cores": int(used),
        "kind": "oracle",
        "sample": f"{heads} of {wf.H} prefill heads ({wf.name}) in {t_f:.1f} s, fp64 NumPy",
        "decode": {"value": dbytes / t_d / 1e9, "unit": "GB/s",
                   "sample": f"{dheads} of {wd.B * wd.H} decode heads ({wd.name}) in {t_d:.1f} s "
                             "(device-to-host copy of each head included)"},
    }


def copy_reference(torch, dev, args):
    """A plain device copy of known size: 1 GiB read + 1 GiB written per launch."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = Event(), Event()
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}), flush=True)
    return 0


def time_gqa(torch, fa, synth, dev, args, traffic):
    """The grouped-query decode (32 query heads over 8 K/V heads, full lengths), timed
    on its own after the step: W warm-up calls, then K calls, each between HIP events."""
    wg = synth.BY_NAME["decode_gqa_b16hq32hkv8_lkv32768_d128_s8"]
    print(f"[bench] generating inputs: {wg.name}", file=sys.stderr, flush=True)
    qg = synth.make_decode_q(wg).to(dev)
    kg, vg = synth.make_decode_kv(wg, device=dev)
    ws = torch.empty(fa.fa_decode_workspace_bytes(wg.B, wg.H, wg.d, wg.num_splits), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        fa.fa_decode_gqa(qg, kg, vg, scale=wg.scale, num_splits=wg.num_splits, workspace=ws)
    torch.cuda.synchronize()
    evs = [[Event() for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record()
        fa.fa_decode_gqa(qg, kg, vg, scale=wg.scale, num_splits=wg.num_splits, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    avg = sum(ms) / len(ms)
    gbytes = synth.decode_bytes(wg)
    gbs = gbytes / (avg * 1e-3) / 1e9
    res = {"workload": wg.name, "B": wg.B, "Hq": wg.H, "Hkv": wg.kv_heads, "Lkv": wg.lkv, "d": wg.d,
           "num_splits": wg.num_splits, "value": round(gbs, 1), "unit": "GB/s", "ms": round(avg, 4),
           "ms_min": round(min(ms), 4), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "algorithmic_bytes": gbytes, "traffic": traffic_bytes(traffic, "gqa")}
    # the same cache in 64-key pages under a seeded random page order
    kp, vp, tbl = synth.paginate(kg, vg, 64, seed=5)
    del kg, vg
    for _ in range(args.warmup):
        fa.fa_decode_paged(qg, kp, vp, tbl, scale=wg.scale, num_splits=wg.num_splits, workspace=ws)
    torch.cuda.synchronize()
    for e in evs:
        e[0].record()
        fa.fa_decode_paged(qg, kp, vp, tbl, scale=wg.scale, num_splits=wg.num_splits, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    pavg = sum(ms) / len(ms)
    pgbs = gbytes / (pavg * 1e-3) / 1e9
    del kp, vp
    paged = {"workload": wg.name + "_paged64", "page_size": 64, "value": round(pgbs, 1), "unit": "GB/s",
             "ms": round(pavg, 4), "ms_min": round(min(ms), 4), "frac_hbm_peak": round(pgbs / HBM_PEAK_GBS, 4),
             "vs_contiguous": round(avg / pavg, 3)}
    return res, paged


def device_facts(torch):
    """Device name, architecture, compute units and the ROCm / HIP versions."""
    props = torch.cuda.get_device_properties(0)
    facts = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": props.multi_processor_count,
             "hip_runtime": torch.version.hip}
    try:
        facts["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        facts["rocm"] = None
    return facts


def sample_gfx_clock(run, seconds=1.0):
    """The shader (gfx) clock while ``run()`` keeps the GPU busy: amd-smi's per-XCD
    current gfx clock, sampled from a second thread about every 0.1 s."""
    import shutil
    import statistics
    import subprocess
    import threading
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(smi):
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run([smi, "metric", "-g", "0", "--clock", "--json"], capture_output=True, text=True,
                                   timeout=5)
                data = json.loads(r.stdout)
                clk = data["gpu_data"][0]["clock"] if isinstance(data, dict) else data[0]["clock"]
                vals = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
                vals = [float(x) for x in vals if isinstance(x, (int, float))]
                if vals and statistics.median(vals) >= 500:  # below the lowest level: idle, between calls
                    samples.append(statistics.median(vals))
            except Exception:
                pass
            stop.wait(0.1)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run()
    stop.set()
    th.join(timeout=10)
    if not samples:
        return None
    return {"median_mhz": statistics.median(samples), "min_mhz": min(samples), "max_mhz": max(samples),
            "samples": len(samples), "source": "amd-smi metric --clock (median over the 8 XCDs per sample) "
                                               "while the Llama-3-shaped prefill ran back to back"}


def time_prefill_workloads(torch, fa, synth, dev, args):
    """Every prefill workload on its own, each call between HIP events: warm (the
    calls back to back, inputs in the caches where they fit) and cold (a 512 MB
    buffer written between calls, outside the timed region); and warm_graph, the
    K calls captured in one HIP graph and timed as one replay (for short calls
    the per-call events also hold the host's launch work)."""
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    res = {}
    for w in synth.WORKLOADS[:4]:
        print(f"[bench] prefill workload: {w.name}", file=sys.stderr, flush=True)
        q, k, v = (t.to(dev) for t in synth.make_prefill(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        call = lambda: fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        ev = [[Event() for _ in range(2)] for _ in range(args.steps)]
        for e in ev:
            e[0].record()
            call()
            e[1].record()
        torch.cuda.synchronize()
        warm = [e[0].elapsed_time(e[1]) for e in ev]
        for i, e in enumerate(ev):
            scrub.fill_(i & 255)
            e[0].record()
            call()
            e[1].record()
        torch.cuda.synchronize()
        cold = [e[0].elapsed_time(e[1]) for e in ev]
        # the same K calls captured once in a HIP graph and replayed between two events:
        # no host work between the calls, so short calls are not timed with their launch
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                call()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = Event(), Event()
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        replay = g0.elapsed_time(g1) / args.steps
        del graph
        flops = synth.prefill_flops(w)
        ent = {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal, "algorithmic_flops": flops,
               "algorithmic_bytes": synth.prefill_bytes(w)}
        for label, ms in (("warm", warm), ("cold", cold), ("warm_graph", [replay])):
            avg = sum(ms) / len(ms)
            tf = flops / (avg * 1e-3) / 1e12
            ent[label] = {"ms": round(avg, 4), "ms_min": round(min(ms), 4), "tflops": round(tf, 2),
                          "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        ent["warm_graph"]["note"] = f"{args.steps} calls replayed from one HIP graph, timed as one replay"
        if w.N * w.H * w.B <= 256:
            ent["note"] = "one workgroup: launch-latency bound, no roofline claim"
        res[w.name] = ent
        del q, k, v, o, lse
    del scrub
    return res


MFMA_FP8_PEAK_TFLOPS = 2 * MFMA_BF16_PEAK_TFLOPS  # dense FP8 matrix rate: twice bf16's


def time_fp8(torch, fa, synth, dev, args):
    """The FP8 prefill on the prefill workload and on the long non-causal one:
    fa_fwd_fp8 on operands fa_quantize_fp8 wrote beforehand, interleaved with the
    bf16 fa_fwd on the same inputs, W + K calls each between HIP events; the
    quantising pass is timed on its own.  ``warm`` times K calls of each back to
    back as well, and ``graph`` K calls of each replayed from a HIP graph (no host
    work between the calls)."""
    res = {}
    for wname in ("llama3_8b_causal_b1h32n4096d128_kboost", "long_noncausal_b1h16n16384d128"):
        w = synth.BY_NAME[wname]
        print(f"[bench] fp8: {w.name}", file=sys.stderr, flush=True)
        q, k, v = (t.to(dev) for t in synth.make_prefill(w))
        packed = fa.fa_quantize_fp8(q, k, v, scale=w.scale)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            fa.fa_fwd_fp8(packed, w.B, w.H, w.N, w.d, causal=w.causal, out=o, lse=lse)
            fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
            fa.fa_quantize_fp8(q, k, v, scale=w.scale, packed=packed)
        torch.cuda.synchronize()
        ev = [[Event() for _ in range(6)] for _ in range(args.steps)]
        for e in ev:
            e[0].record()
            fa.fa_fwd_fp8(packed, w.B, w.H, w.N, w.d, causal=w.causal, out=o, lse=lse)
            e[1].record()
            e[2].record()
            fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
            e[3].record()
            e[4].record()
            fa.fa_quantize_fp8(q, k, v, scale=w.scale, packed=packed)
            e[5].record()
        torch.cuda.synchronize()
        f8, bf, qz = (sum(e[a].elapsed_time(e[a + 1]) for e in ev) / len(ev) for a in (0, 2, 4))
        # each call also K times back to back (warm caches, the same power state for both)
        warm = {}
        for label, call in (("fp8", lambda: fa.fa_fwd_fp8(packed, w.B, w.H, w.N, w.d, causal=w.causal, out=o,
                                                           lse=lse)),
                            ("bf16", lambda: fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse))):
            call()
            torch.cuda.synchronize()
            evw = [[Event() for _ in range(2)] for _ in range(args.steps)]
            for e in evw:
                e[0].record()
                call()
                e[1].record()
            torch.cuda.synchronize()
            warm[label] = sum(e[0].elapsed_time(e[1]) for e in evw) / len(evw)
            # and K calls captured in one HIP graph, timed as one replay (no host work between them)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(args.steps):
                    call()
            graph.replay()
            torch.cuda.synchronize()
            g0, g1 = Event(), Event()
            g0.record()
            graph.replay()
            g1.record()
            torch.cuda.synchronize()
            warm[label + "_graph"] = g0.elapsed_time(g1) / args.steps
            del graph
        flops = synth.prefill_flops(w)
        tf = flops / (f8 * 1e-3) / 1e12
        res[w.name] = {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(f8, 4),
                       "frac_mfma_fp8_peak": round(tf / MFMA_FP8_PEAK_TFLOPS, 4), "bf16_ms": round(bf, 4),
                       "speedup_vs_bf16": round(bf / f8, 3), "quantize_ms": round(qz, 4),
                       "warm": {"ms": round(warm["fp8"], 4), "bf16_ms": round(warm["bf16"], 4),
                                "speedup_vs_bf16": round(warm["bf16"] / warm["fp8"], 3),
                                "note": f"{args.steps} calls of each back to back"},
                       "graph": {"ms": round(warm["fp8_graph"], 4), "bf16_ms": round(warm["bf16_graph"], 4),
                                 "speedup_vs_bf16": round(warm["bf16_graph"] / warm["fp8_graph"], 3),
                                 "note": f"{args.steps} calls of each captured in a HIP graph, timed as one replay"}}
    return res


def time_sparse(torch, fa, synth, dev, args, traffic):
    """Block-sparse forward against the dense forward on the long workload, each timed
    W + K calls between HIP events, interleaved."""
    ws_ = synth.BY_NAME["long_noncausal_b1h16n16384d128"]
    print(f"[bench] block sparse: {ws_.name}", file=sys.stderr, flush=True)
    q, k, v = (t.to(dev) for t in synth.make_prefill(ws_))
    mask = synth.make_block_mask(ws_, 0.1)
    md = mask.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((ws_.B, ws_.H, ws_.N), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        fa.fa_fwd_block_sparse(q, k, v, md, scale=ws_.scale, out=o, lse=lse)
        fa.fa_fwd(q, k, v, scale=ws_.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    ev = [[Event() for _ in range(4)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        fa.fa_fwd_block_sparse(q, k, v, md, scale=ws_.scale, out=o, lse=lse)
        e[1].record()
        e[2].record()
        fa.fa_fwd(q, k, v, scale=ws_.scale, out=o, lse=lse)
        e[3].record()
    torch.cuda.synchronize()
    sp = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev)
    dn = sum(e[2].elapsed_time(e[3]) for e in ev) / len(ev)
    flops = synth.block_sparse_flops(ws_, mask)
    kept = float(mask.float().mean())
    tf = flops / (sp * 1e-3) / 1e12
    res = {"workload": ws_.name + "_blocksparse", "mask": "own + first key block, 10 % of the rest (seeded)",
           "kept_blocks": round(kept, 4), "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(sp, 4),
           "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "dense_ms": round(dn, 4),
           "speedup_vs_dense": round(dn / sp, 2), "ideal_speedup": round(1 / kept, 2), "algorithmic_flops": flops,
           "traffic": traffic_bytes(traffic, "sparse")}
    if args.only == "sparse" and args.no_bwd_atomic:  # counter runs: the forward alone
        return res
    # the backward of both, on the forwards' own O and L and a seeded dO
    do = synth.make_prefill_grad(ws_).to(dev)
    o_s, lse_s = fa.fa_fwd_block_sparse(q, k, v, md, scale=ws_.scale)
    o_d, lse_d = fa.fa_fwd(q, k, v, scale=ws_.scale)
    wsp = torch.empty(fa.fa_bwd_workspace_bytes(ws_.B, ws_.H, ws_.N), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        fa.fa_bwd_block_sparse(q, k, v, o_s, lse_s, do, md, scale=ws_.scale, workspace=wsp)
        fa.fa_bwd(q, k, v, o_d, lse_d, do, scale=ws_.scale, workspace=wsp)
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        fa.fa_bwd_block_sparse(q, k, v, o_s, lse_s, do, md, scale=ws_.scale, workspace=wsp)
        e[1].record()
        e[2].record()
        fa.fa_bwd(q, k, v, o_d, lse_d, do, scale=ws_.scale, workspace=wsp)
        e[3].record()
    torch.cuda.synchronize()
    bsp = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev)
    bdn = sum(e[2].elapsed_time(e[3]) for e in ev) / len(ev)
    bflops = 2.5 * flops  # the five products of the backward against the forward's two
    res["backward"] = {"value": round(bflops / (bsp * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms": round(bsp, 4),
                       "dense_ms": round(bdn, 4), "speedup_vs_dense": round(bdn / bsp, 2),
                       "note": "fa_bwd_block_sparse against fa_bwd on the same workload; five products of the kept blocks"}
    return res


def time_bwd(torch, fa, synth, dev, args, wf, q, k, v, traffic):
    """The backward on the prefill workload, timed on its own: the forward's O and L
    and a seeded dO, W warm-up calls, then K calls, each between HIP events."""
    print(f"[bench] backward: {wf.name}", file=sys.stderr, flush=True)
    do = synth.make_prefill_grad(wf).to(dev)
    o, lse = fa.fa_fwd(q, k, v, scale=wf.scale, causal=wf.causal)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(wf.B, wf.H, wf.N), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        fa.fa_bwd(q, k, v, o, lse, do, scale=wf.scale, causal=wf.causal, workspace=ws)
    torch.cuda.synchronize()
    evs = [[Event() for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record()
        fa.fa_bwd(q, k, v, o, lse, do, scale=wf.scale, causal=wf.causal, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    avg = sum(ms) / len(ms)
    flops = synth.bwd_flops(wf)
    tf = flops / (avg * 1e-3) / 1e12
    res = {"workload": wf.name, "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(avg, 4),
           "ms_min": round(min(ms), 4), "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
           "algorithmic_flops": flops,
           "algorithmic_bytes": float(wf.B * wf.H * (16 * wf.N * wf.d + 4 * wf.N)),
           "traffic": traffic_bytes(traffic, "bwd"),
           "note": "two kernels per call (dQ, which also forms the per-row L and D; then dK, dV); the dQ pass "
                   "recomputes S and dP, so the matrix cores run 7/5 of the counted FLOPs"}
    if args.no_bwd_atomic:
        return res
    # the one-pass form with atomic dQ, timed the same way for comparison
    wsa = torch.empty(fa.fa_bwd_atomic_workspace_bytes(wf.B, wf.H, wf.N, wf.d), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        fa.fa_bwd_atomic(q, k, v, o, lse, do, scale=wf.scale, causal=wf.causal, workspace=wsa)
    torch.cuda.synchronize()
    for e in evs:
        e[0].record()
        fa.fa_bwd_atomic(q, k, v, o, lse, do, scale=wf.scale, causal=wf.causal, workspace=wsa)
        e[1].record()
    torch.cuda.synchronize()
    ms_a = [e[0].elapsed_time(e[1]) for e in evs]
    avg_a = sum(ms_a) / len(ms_a)
    res["atomic"] = {"value": round(flops / (avg_a * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms": round(avg_a, 4),
                     "note": "fa_bwd_atomic: one key-block pass, dQ added up with fp32 atomics"}
    return res


def main():
    args = parse()
    global EVENT_KIND
    EVENT_KIND = args.events
    if args.make_traffic:
        return make_traffic(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path; the single-GPU figure is the measurement.", file=sys.stderr)
        return 2

    import torch
    import exact_attention_31_amd as fa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "copy":
        return copy_reference(torch, dev, args)

    wf = synth.BY_NAME["llama3_8b_causal_b1h32n4096d128_kboost"]
    if args.prefill:
        if args.only != "fwd":
            print("--prefill goes with --only fwd", file=sys.stderr)
            return 2
        wf = synth.BY_NAME[args.prefill]
    wd = synth.BY_NAME["decode_b16h32_lkv32768_d128_s64"]
    do_f = args.only in ("all", "fwd")
    do_d = args.only in ("all", "decode")
    print(f"[bench] generating inputs: {wf.name}, {wd.name}", file=sys.stderr, flush=True)
    q = k = v = o = lse = qd = kd = vd = ws = None
    if do_f or args.only in ("all", "bwd"):
        q, k, v = (t.to(dev) for t in synth.make_prefill(wf))
        o = torch.empty_like(q)
        lse = torch.empty((wf.B, wf.H, wf.N), dtype=torch.float32, device=dev)
    if do_d:
        qd = synth.make_decode_q(wd).to(dev)
        kd, vd = synth.make_decode_kv(wd, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(wd.B, wd.H, wd.d, wd.num_splits), dtype=torch.uint8,
                         device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if do_f:
            fa.fa_fwd(q, k, v, scale=wf.scale, causal=wf.causal, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        if do_d:
            fa.fa_decode(qd, kd, vd, scale=wd.scale, num_splits=wd.num_splits, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warm-up done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    evs = [[Event() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs] if do_f else []
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs] if do_d else []

    flops = synth.prefill_flops(wf)
    fbytes = synth.prefill_bytes(wf)
    dbytes = synth.decode_bytes(wd)
    f_avg = sum(fwd_ms) / len(fwd_ms) if fwd_ms else None
    d_avg = sum(dec_ms) / len(dec_ms) if dec_ms else None

    traffic = {}
    if os.path.exists(args.traffic):
        try:
            traffic = json.load(open(args.traffic))
        except Exception:
            traffic = {}

    out = {
        "metric": METRIC,
        "value": round(flops / (f_avg * 1e-3) / 1e12, 2) if f_avg else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wf.name} + {wd.name}",
            "prefill": {"B": wf.B, "H": wf.H, "N": wf.N, "d": wf.d, "causal": wf.causal, "scale": wf.scale},
            "decode": {"B": wd.B, "H": wd.H, "Lkv": wd.lkv, "d": wd.d, "num_splits": wd.num_splits},
            "parallelism": "single GPU",
        },
    }
    out["device"] = device_facts(torch)
    out["timing"] = ("HIP events on the launch stream, created with hipEventDisableSystemFence" if args.events == "nofence"
                     else "torch.cuda.Event on the launch stream (system-scope fence at each record)")
    if f_avg:
        tf = flops / (f_avg * 1e-3) / 1e12
        out["prefill"] = {"ms": round(f_avg, 4), "ms_min": round(min(fwd_ms), 4), "tflops": round(tf, 2),
                          "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "caches": "cold: each call follows the decode's 8.6 GB stream" if do_d else "warm"}
        out["roofline"] = {"kernel": f"fa_fwd_kernel<{wf.d},{str(wf.causal).lower()}>", "bound": "mfma",
                           "achieved": round(tf, 2),
                           "peak": round(MFMA_BF16_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                           "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                           "traffic": None if args.prefill else traffic_bytes(traffic, "fwd"),
                           "algorithmic_bytes": fbytes}
    if d_avg:
        gbs = dbytes / (d_avg * 1e-3) / 1e9
        out["decode"] = {"value": round(gbs, 1), "unit": "GB/s", "ms": round(d_avg, 4), "ms_min": round(min(dec_ms), 4),
                         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        out["roofline_decode"] = {"kernel": "fa_decode_split_kernel<128> + fa_decode_combine_kernel<128>",
                                  "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "traffic": traffic_bytes(traffic, "decode"), "algorithmic_bytes": dbytes}
    if args.only == "all" and f_avg:
        out["device"]["gfx_clock_during_prefill"] = sample_gfx_clock(
            lambda: (fa.fa_fwd(q, k, v, scale=wf.scale, causal=wf.causal, out=o, lse=lse), torch.cuda.synchronize()))
    if args.only in ("all", "workloads"):
        out["prefill_workloads"] = time_prefill_workloads(torch, fa, synth, dev, args)
    if args.only in ("all", "gqa"):
        out["decode_gqa"], out["decode_paged"] = time_gqa(torch, fa, synth, dev, args, traffic)
    if args.only in ("all", "bwd"):
        out["backward"] = time_bwd(torch, fa, synth, dev, args, wf, q, k, v, traffic)
    if args.only in ("all", "sparse"):
        out["block_sparse"] = time_sparse(torch, fa, synth, dev, args, traffic)
    if args.only in ("all", "fp8"):
        out["fp8"] = time_fp8(torch, fa, synth, dev, args)
    if not args.no_cpu_baseline and args.only == "all":
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wf, wd, q, k, v, qd, kd, vd, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
