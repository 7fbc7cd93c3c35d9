#!/usr/bin/env python3
"""Benchmark of the fused W4A4 + INT8-outlier linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--m M] [--norm]

The default workload is the largest prefill projection (the Llama-65B
down_proj, M = 8192, K = 22016, N = 8192, per-row scales, 256 INT8 outlier
channels); --workload qproj|upproj|decode|tiny selects the others.

One step is one pass of the layer's run-time path over one batch: the
activation producer (reorder + INT4/INT8 quantize, ``w4a4_quant_reorder_act``)
then the mixed-precision GEMM with its fp32 epilogue (``w4a4_outlier_gemm``);
together they are exactly what ``w4a4_quant_gemm`` launches. Weights are
quantized and packed once before timing, as the layer does offline. With
``--norm`` the producer is the one fused with the preceding RMSNorm
(``w4a4_rmsnorm_quant_reorder_act``, gamma ~ 1 + N(0, 0.1), eps = 1e-6), and
the step is what ``w4a4_rmsnorm_quant_gemm`` launches.

Inputs are seeded synthetic tensors already resident in HBM. Buffer sets
(X, packed W, quantized activations, Y) are rotated so that the working set
of consecutive steps exceeds 512 MB and the 256 MB Infinity Cache cannot
serve them.

Prints one JSON line. ``value`` is the whole-step throughput in TOPS
(2 M N K integer ops per step). ``roofline`` describes the dominant kernel,
the GEMM: its algorithmic ops (or bytes, for memory-bound decode shapes) per
launch divided by its mean duration, measured with HIP events recorded on
the launch stream around the GEMM launches inside the timed region: every
launch when a step takes longer than LONG_STEP_MS, else every EVENT_EVERY-th
(an event pair costs about 5 us, which short steps would carry); the line
reports their mean, p10, p50 and p90. The producer is timed by events in a
short loop after it, so that no event sits between the two kernels of a timed
step. The shader clock is sampled during the timed region (amdsmi, else
rocm-smi) and reported with the line, since the matrix-core rate on this chip
depends on the clock it holds under load.
``cpu_baseline`` times the CPU oracle on the host cores on a bounded row
sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5033.2      # 256 CU x 2.4 GHz x 8192 dense int8 ops / clk / CU
PEAK_FP6_TOPS = 10066.3      # 256 CU x 2.4 GHz x 16384 dense fp6 (f8f6f4) ops / clk / CU
PEAK_HBM_GBS = 8000.0        # HBM3E
ROTATE_BYTES = 512 << 20
EVENT_EVERY = 8              # timed steps per HIP event pair around the GEMM (short steps)
LONG_STEP_MS = 0.2           # steps at least this long get an event pair every step

from mixed_precision_integer_amd import workloads as wl  # noqa: E402

WORKLOADS = {"tiny": wl.TINY, "qproj": wl.QPROJ_7B, "upproj": wl.UPPROJ_7B,
             "decode": wl.DECODE_65B, "downproj": wl.DOWNPROJ_65B}


def work_counts(w, M, norm=False, fp6=False):
    """Algorithmic ops and bytes of one layer call (zero padding not counted);
    the norm-fused producer also reads the K fp16 norm weights. The INT4 head
    is half a byte per code, or 6 bits on the FP6 path (its u6 operands)."""
    N, K, n_out, K_n = w.N, w.K, w.n_out, w.K_n
    G = (K_n // w.group if w.group else 1) if K_n else 0
    ops = 2 * M * N * K
    code = 0.75 if fp6 else 0.5
    w_bytes = N * K_n * code + N * n_out + 4 * N * G + 4 * N
    a_bytes = M * K_n * code + M * n_out + 4 * M * G + 4 * M
    gemm_bytes = w_bytes + a_bytes + 2 * M * N
    producer_bytes = 2 * M * K + a_bytes + (2 * K if norm else 0)
    # one launch (quantizer inside the GEMM): fp16 tokens and the permutation
    # (and the norm weights) in place of the codes
    one_launch_bytes = w_bytes + 2 * M * K + 4 * K + (2 * K if norm else 0) + 2 * M * N
    return ops, gemm_bytes, producer_bytes, one_launch_bytes


class ClockSampler:
    """Samples the GPU's current shader clock (MHz) on a host thread while the
    timed region runs; reports the median of the readings and where they came
    from. Nothing here touches the GPU's work."""

    def __init__(self, period_s=0.005):
        import threading
        self.period_s, self.samples, self.source = period_s, [], None
        self._stop = threading.Event()
        self._thread = None
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handle = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                info = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
                return float(info.get("clk", info.get("cur_clk")))
            read()
            self._read, self.source = read, "amdsmi_get_clock_info(GFX)"
        except Exception:
            self._read = None
        if self._read is None:
            self._read, self.source = self._rocm_smi, "rocm-smi --showclocks"

    @staticmethod
    def _rocm_smi():
        import re
        import subprocess
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=10).stdout
        m = re.search(r"sclk.*?\((\d+)Mhz\)", out, re.I)
        return float(m.group(1)) if m else None

    def _loop(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v:
                    self.samples.append(v)
            except Exception:
                pass
            self._stop.wait(self.period_s)

    def __enter__(self):
        import threading
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)

    def report(self):
        if not self.samples:
            return {"mhz": None, "samples": 0, "source": self.source}
        return {"mhz": float(np.median(self.samples)), "min_mhz": float(min(self.samples)),
                "max_mhz": float(max(self.samples)), "samples": len(self.samples), "source": self.source}


def profile_record(workload_name, M, kernel):
    """The committed counter record of this kernel on this workload
    (profiles/gemm_traffic.json), if it was taken on the kernel's current
    sources; else None."""
    from mixed_precision_integer_amd import profile_summary as ps
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    for key, rec in json.load(open(path)).items():
        recorded = rec.get("kernel", "").split("(")[0].split("::")[-1]
        if key != ps.traffic_key(workload_name, M, recorded):
            continue
        if recorded != kernel and not recorded.startswith(kernel + "<"):
            continue
        if rec.get("gemm_sources_sha256_16") == ps.gemm_source_digest(recorded):
            return rec
    return None


def traffic_record(workload_name, M, kernel):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs
    (profiles/gemm_traffic.json), if they were taken of this kernel on its
    current sources; else None."""
    rec = profile_record(workload_name, M, kernel)
    return rec.get("hbm_bytes_per_launch") if rec else None


def sclk_report(clock, rec, kernel):
    """The GEMM kernel's achieved shader clock: GRBM_GUI_ACTIVE / 8 XCDs / its
    duration, from the committed counter run of this kernel and workload (the
    SMU's clock readings taken during the timed region are reported beside
    it; on this machine they do not follow the shader clock)."""
    smu = clock.report()
    out = {"mhz": None, "source": None, "smu_samples": smu}
    if rec and rec.get("sclk_mhz"):
        out["mhz"] = rec["sclk_mhz"]
        out["source"] = f"GRBM_GUI_ACTIVE / 8 XCDs / duration of {kernel}, profiles/{rec.get('profile')}"
    return out


def cpu_baseline(w, X, W, outliers, budget_s, gamma=None, eps=0.0):
    """The CPU oracle on the host: producer (after the RMSNorm when gamma is
    given) + integer GEMM + fp64 dequant for a row sample of X against all N
    output channels (weights pre-quantized)."""
    import oracle
    perm = oracle.make_perm(w.K, outliers)
    qw = oracle.quantize_rows(W, perm, w.n_out, w.group)
    nn = np.arange(w.N, dtype=np.int32)

    def run(rows):
        t0 = time.perf_counter()
        if gamma is None:
            qa = oracle.quantize_rows(X[:rows], perm, w.n_out, w.group)
        else:
            qa = oracle.rmsnorm_quantize_rows(X[:rows], gamma, eps, perm, w.n_out, w.group)
        mm = np.repeat(np.arange(rows, dtype=np.int32), w.N)
        oracle.linear_at(qa, qw, w.group, mm, np.tile(nn, rows))
        return time.perf_counter() - t0

    M = X.shape[0]
    r0 = min(M, 2)
    t0 = run(r0)
    rows = int(min(M, max(r0, math.floor(r0 * budget_s / max(t0, 1e-6)))))
    t = run(rows)
    return {
        "value": 2.0 * rows * w.N * w.K / t / 1e12,
        "unit": "TOPS",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": (f"{rows} of {M} token rows x all {w.N} output channels: "
                   f"{'RMSNorm + ' if gamma is not None else ''}producer, integer "
                   f"GEMM and fp64 dequant (weights quantized beforehand); {t:.1f} s"),
    }


SELECT_WORKLOADS = {
    # name: (calibration rows, K, n_out): 16 x 2048 tokens of a 4096-channel
    # input, and 4 x 2048 tokens of the 65B down_proj's 22016 channels
    "qproj": (32768, 4096, 128),
    "downproj": (8192, 22016, 256),
}


def select_bench(torch, w4, args):
    """Offline outlier-channel selection (w4a4_select_outliers): HBM-bound
    column absmax over a synthetic calibration batch plus the one-workgroup
    select. Prints its own JSON line."""
    rows, K, n_out = SELECT_WORKLOADS[args.select_outliers]
    X, _, _ = wl.draw(rows, 1, K, n_out, seed=rows + K, outlier_factor=30.0)
    dev = torch.device("cuda:0")
    n_sets = max(2, math.ceil(ROTATE_BYTES / (rows * K * 2)))
    Xs = [torch.from_numpy(X).to(dev) for _ in range(n_sets)]
    ws = torch.empty(max(w4.select_outliers_workspace_bytes(rows, K), 256), dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        w4.select_outliers(Xs[i % n_sets], n_out, workspace=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, e in enumerate(ev):
        e[0].record()
        w4.select_outliers(Xs[i % n_sets], n_out, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    nbytes = 2.0 * rows * K
    ach = nbytes / (call_ms * 1e-3) / 1e9
    idx, _ = w4.select_outliers(Xs[0], n_out, workspace=ws)
    out = {
        "metric": "outlier-channel selection GB/s (calibration absmax + top-n select) & % HBM",
        "value": ach, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u16", "data": "synthetic",
        "config": {"workload": f"select_outliers_{args.select_outliers}_rows{rows}_k{K}_n{n_out}",
                   "rows": rows, "K": K, "n_out": n_out, "buffer_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "colmax_kernel + fold_kernel + select_kernel (one call)"},
    }
    if not args.no_cpu_baseline:
        import oracle
        r = max(64, min(rows, int(rows * 0.25)))
        t = time.perf_counter()
        want = oracle.select_outliers(X[:r], n_out)
        dt = time.perf_counter() - t
        out["cpu_baseline"] = {"value": 2.0 * r * K / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{r} of {rows} calibration rows (numpy absmax + lexsort), {dt:.2f} s"}
        del want
    print(json.dumps(out), flush=True)
    return idx


W4A8_WORKLOADS = {
    # name: (M, N, K, group): the Llama-7B q_proj prefill with 128-channel
    # weight groups, and up_proj with one weight scale per output channel
    "qproj": (2048, 4096, 4096, 128),
    "upproj": (4096, 11008, 4096, 0),
}


def w4a8_bench(torch, w4, args):
    """W4A8 layer step: per-token INT8 activation producer, then the W4A8
    GEMM (weights packed before timing). Prints its own JSON line; the
    roofline is the GEMM's."""
    M, N, K, group = W4A8_WORKLOADS[args.w4a8]
    X, W, _ = wl.draw(M, N, K, 0, seed=M + N + group)
    dev = torch.device("cuda:0")
    wq = w4.pack_int4_weights_w4a8(torch.from_numpy(W).to(dev), group)
    one = M * K * 3 + N * K // 2 + M * N * 2
    n_sets = max(2, math.ceil(ROTATE_BYTES / one) + 1)
    sets = []
    for _ in range(n_sets):
        Xd = torch.from_numpy(X).to(dev)
        a = w4.quant_act_int8(Xd)
        wc = w4.W4A8Operand(wq.q.clone(), wq.s.clone(), K, group)
        sets.append((Xd, a, wc, torch.empty((M, N), dtype=torch.float16, device=dev)))
    L = w4.lib()
    stream = w4._stream()

    def produce(st):
        Xd, a = st[0], st[1]
        rc = L.w4a4_quant_reorder_act(Xd.data_ptr(), K, None, M, K, K, 0, None, a.q.data_ptr(), None,
                                      a.s.data_ptr(), stream)
        if rc:
            raise SystemExit(f"producer failed: {rc}")

    def gemm(st):
        a, wc, y = st[1], st[2], st[3]
        rc = L.w4a4_w4a8_gemm(a.q.data_ptr(), a.s.data_ptr(), wc.q.data_ptr(), wc.s.data_ptr(), M, N, K,
                              group, y.data_ptr(), N, stream)
        if rc:
            raise SystemExit(f"W4A8 GEMM failed: {rc}")

    for i in range(args.warmup):
        produce(sets[i % n_sets])
        gemm(sets[i % n_sets])
    torch.cuda.synchronize()
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in range(0, args.steps, EVENT_EVERY)}
    t0 = time.perf_counter()
    for i in range(args.steps):
        produce(sets[i % n_sets])
        e = ev.get(i)
        if e:
            e[0].record()
        gemm(sets[i % n_sets])
        if e:
            e[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gemm_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev.values()]))
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(min(args.steps, 50))]
    for i, e in enumerate(pev):
        e[0].record()
        produce(sets[i % n_sets])
        e[1].record()
        gemm(sets[i % n_sets])
    torch.cuda.synchronize()
    prod_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pev]))
    ms_step = (t1 - t0) * 1e3 / args.steps
    ops = 2.0 * M * N * K
    G = K // group if group else 1
    prod_bytes = 2 * M * K + M * K + 4 * M
    ach = ops / (gemm_ms * 1e-3) / 1e12
    out = {
        "metric": "W4A8 linear TOPS & % INT8-MFMA peak",
        "value": ops / (ms_step * 1e-3) / 1e12, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"w4a8_{args.w4a8}_m{M}_n{N}_k{K}_g{group}", "M": M, "N": N, "K": K,
                   "group": group, "buffer_sets": n_sets},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": ach / PEAK_INT8_TOPS, "traffic": None, "kernel": "gemm_w4a8_kernel"},
        "kernels": {"producer_us": prod_ms * 1e3, "producer_GBps": prod_bytes / (prod_ms * 1e-3) / 1e9,
                    "gemm_us": gemm_ms * 1e3, "gemm_TOPS": ach,
                    "gemm_GBps": (N * K / 2 + 4 * N * G + M * K + 4 * M + 2 * M * N) / (gemm_ms * 1e-3) / 1e9},
    }
    if not args.no_cpu_baseline:
        import oracle
        _, qw = oracle.w4a8_quantize(X[:1], W, group)          # weights quantized beforehand
        nn = np.arange(N, dtype=np.int32)

        def run(rows):
            t = time.perf_counter()
            qa, _ = oracle.w4a8_quantize(X[:rows], W[:1], group)
            oracle.w4a8_linear_at(qa, qw, group, np.repeat(np.arange(rows, dtype=np.int32), N),
                                  np.tile(nn, rows))
            return time.perf_counter() - t

        dt0 = run(8)
        r = int(min(M, max(8, 8 * args.cpu_budget / max(dt0, 1e-6))))
        dt = run(r)
        out["cpu_baseline"] = {"value": 2.0 * r * N * K / dt / 1e12, "unit": "TOPS",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{r} of {M} token rows x all {N} output channels (weights "
                                         f"quantized beforehand), {dt:.1f} s"}
    print(json.dumps(out), flush=True)


KV_WORKLOADS = {
    # name: (tokens, heads, head dim, bits): a Llama-65B-style prefill of
    # 8 x 2048 tokens appended to the key (or value) cache
    "int4": (16384, 64, 128, 4),
    "int8": (16384, 64, 128, 8),
}


def kv_bench(torch, w4, args):
    """Low-bit KV cache: a step quantizes one tensor's new tokens into the
    cache (w4a4_kv_quant) and gathers them back (w4a4_kv_dequant). Prints its
    own JSON line; value = bytes both calls must move / step time."""
    T, H, D, bits = KV_WORKLOADS[args.kv]
    rng = np.random.default_rng(T + bits)
    X = (rng.standard_normal((T, H * D), dtype=np.float32)
         * rng.choice([0.05, 1.0, 30.0], (T, H)).repeat(D, axis=1).astype(np.float32)).astype(np.float16)
    dev = torch.device("cuda:0")
    n_sets = max(2, math.ceil(ROTATE_BYTES / (T * H * D * 2 * 2)))
    slots = torch.from_numpy(np.random.default_rng(1).permutation(2 * T)[:T].astype(np.int32)).to(dev)
    sets = [(torch.from_numpy(X).to(dev), w4.KVCache(2 * T, H, D, bits, dev),
             torch.empty((T, H * D), dtype=torch.float16, device=dev)) for _ in range(n_sets)]
    for i in range(args.warmup):
        x, c, y = sets[i % n_sets]
        c.store(x, slots)
        c.load(slots, out=y)
    torch.cuda.synchronize()
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in range(0, args.steps, EVENT_EVERY)}
    t0 = time.perf_counter()
    for i in range(args.steps):
        x, c, y = sets[i % n_sets]
        e = ev.get(i)
        if e:
            e[0].record()
        c.store(x, slots)
        if e:
            e[1].record()
        c.load(slots, out=y)
        if e:
            e[2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    q_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev.values()]))
    d_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev.values()]))
    code_bytes = T * H * (D * bits // 8 + 4)
    q_bytes = T * H * D * 2 + code_bytes + 4 * T
    d_bytes = code_bytes + T * H * D * 2 + 4 * T
    ms_step = (t1 - t0) * 1e3 / args.steps
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    out = {
        "metric": "low-bit KV cache GB/s (quantize into the cache + gather back) & % HBM",
        "value": (q_bytes + d_bytes) / (ms_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": f"int{bits}", "data": "synthetic",
        "config": {"workload": f"kv_cache_t{T}_h{H}_d{D}_int{bits}", "T": T, "H": H, "D": D, "bits": bits,
                   "buffer_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": q_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": q_gbs / PEAK_HBM_GBS, "traffic": None, "kernel": f"kv_quant_kernel<16, {bits}>"},
        "kernels": {"quant_us": q_ms * 1e3, "quant_GBps": q_gbs, "dequant_us": d_ms * 1e3,
                    "dequant_GBps": d_bytes / (d_ms * 1e-3) / 1e9},
    }
    if not args.no_cpu_baseline:
        import oracle
        r = min(T, 2048)
        t = time.perf_counter()
        q, s = oracle.kv_quantize(X[:r].reshape(r, H, D), bits)
        oracle.kv_dequantize(q, s)
        dt = time.perf_counter() - t
        out["cpu_baseline"] = {"value": r * H * D * 2 * 2 / dt / 1e9, "unit": "GB/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{r} of {T} tokens, quantize + dequantize, {dt:.2f} s"}
    print(json.dumps(out), flush=True)


def copy_probe(torch, nbytes, steps, warmup):
    """A plain copy of known size: it reads and writes exactly `nbytes` of HBM
    per launch, so the hardware counters it produces give the scale from
    FETCH_SIZE / WRITE_SIZE to bytes."""
    dev = torch.device("cuda:0")
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = [torch.empty_like(src) for _ in range(2)]
    for i in range(warmup):
        dst[i % 2].copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        dst[i % 2].copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / max(steps, 1)
    print(json.dumps({"copy_probe_bytes": nbytes, "us_per_copy": us,
                      "GBps": 2 * nbytes / us / 1e3}), flush=True)


def read_probe(torch, sizes_mib, steps):
    """A hand-written streaming read (probe/read_probe.hip, libw4a4_probe.so)
    of buffers of each size, cold: the launches rotate over buffer sets of more
    than 1.5 GiB, so that no set is still in the 256 MB last-level cache when it
    is read again. Swept over workgroup counts, loads of 16 bytes in flight
    per lane and plain or non-temporal loads; one JSON line per setting (median
    of `steps` launches, each bracketed by HIP events on its stream), then the
    best per size."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mixed_precision_integer_amd", "libw4a4_probe.so"))
    lib.w4a4_read_probe.restype = ctypes.c_int32
    lib.w4a4_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.w4a4_read_probe_out_words.restype = ctypes.c_int64
    lib.w4a4_read_probe_out_words.argtypes = [ctypes.c_int32]
    dev = torch.device("cuda:0")
    wgs_list, depths = (256, 512, 1024, 2048, 4096), (1, 2, 4, 8, 16)
    out = torch.empty(int(lib.w4a4_read_probe_out_words(max(wgs_list))), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    best = {}
    for mib in sizes_mib:
        nbytes = mib << 20
        n_sets = max(2, -(-(3 << 29) // nbytes))
        bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        k = 0
        for wgs in wgs_list:
            for depth in depths:
                for nt in (0, 1):
                    ts = []
                    for it in range(steps + 2):
                        b = bufs[k % n_sets]
                        k += 1
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        rc = lib.w4a4_read_probe(b.data_ptr(), nbytes, wgs, depth, nt, out.data_ptr(),
                                                 ctypes.c_void_p(stream.cuda_stream))
                        e1.record(stream)
                        if rc != 0:
                            raise SystemExit(f"w4a4_read_probe returned {rc}")
                        torch.cuda.synchronize()
                        if it >= 2:
                            ts.append(e0.elapsed_time(e1) * 1e3)
                    us = float(np.median(ts))
                    rec = {"read_probe_bytes": nbytes, "workgroups": wgs, "loads_in_flight_per_lane": depth,
                           "nontemporal": bool(nt), "us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)}
                    print(json.dumps(rec), flush=True)
                    if mib not in best or rec["GBps"] > best[mib]["GBps"]:
                        best[mib] = rec
        del bufs
        torch.cuda.empty_cache()
    print(json.dumps({"read_probe_best": list(best.values())}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="downproj", choices=sorted(WORKLOADS))
    ap.add_argument("--m", type=int, default=None, help="token rows (decode sweep)")
    ap.add_argument("--custom", default=None,
                    help="M,N,K,n_out,group: a synthetic shape instead of a named workload")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select-outliers", default=None, choices=sorted(SELECT_WORKLOADS),
                    help="instead of the layer, time the offline outlier-channel selection")
    ap.add_argument("--w4a8", default=None, choices=sorted(W4A8_WORKLOADS),
                    help="instead of the W4A4 layer, time the W4A8 layer (INT8 producer + W4A8 GEMM)")
    ap.add_argument("--kv", default=None, choices=sorted(KV_WORKLOADS),
                    help="instead of the layer, time the low-bit KV cache (quantize + gather)")
    ap.add_argument("--path", default="auto", choices=("auto", "fp6", "i8"),
                    help="prefill GEMM path: fp6 (INT4 codes q as FP6 E2M3 q / 8 on the FP6 matrix cores) or i8 "
                         "(widened nibbles on the i8 matrix cores); auto takes fp6 where it applies "
                         "and its tiles fill every CU (with --norm too)")
    ap.add_argument("--norm", action="store_true",
                    help="producer fused with the preceding RMSNorm (eps 1e-6)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the layer, time a plain device-to-device copy of this many "
                         "MiB (reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--read-probe-mib", type=str, default="",
                    help="instead of the layer, sweep the hand-written streaming-read probe over these "
                         "buffer sizes (comma-separated MiB; cold buffers)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards by rows or columns with no communication, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mixed_precision_integer_amd as w4

    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib << 20, args.steps, args.warmup)
        return
    if args.read_probe_mib:
        read_probe(torch, [int(v) for v in args.read_probe_mib.split(",")], max(3, min(args.steps, 15)))
        return
    if args.select_outliers:
        select_bench(torch, w4, args)
        return
    if args.w4a8:
        w4a8_bench(torch, w4, args)
        return
    if args.kv:
        kv_bench(torch, w4, args)
        return

    w = WORKLOADS[args.workload]
    if args.custom:
        cm, cn, ck, co, cg = (int(v) for v in args.custom.split(","))
        w = wl.Workload(f"custom_m{cm}_n{cn}_k{ck}_o{co}_g{cg}", cm, cn, ck, co, cg, 7, "normal",
                        30.0, 0.02)
    M = args.m if args.m is not None else w.M
    X, W, outliers = wl.draw_workload(w, M if M <= w.M else None)
    if M > X.shape[0]:
        raise SystemExit(f"--m {M} exceeds the workload's {w.M} rows")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    perm = torch.from_numpy(w4.make_perm(w.K, outliers)).to(dev)
    Xd = torch.from_numpy(X).to(dev)
    wq = w4.pack_int4_weights(torch.from_numpy(W).to(dev), perm, w.n_out, w.group)

    def clone_op(op):
        return w4.QuantizedOperand(*[None if t is None else t.clone() for t in op[:4]], *op[4:])

    one_set = (Xd.numel() * 2 + M * w.N * 2 + sum(t.numel() * t.element_size()
                                                   for t in wq[:4] if t is not None) * 2)
    n_sets = max(2, math.ceil(ROTATE_BYTES / one_set) + 1)
    norm = None
    if args.norm:
        norm = (torch.from_numpy(wl.draw_norm_weight(w.K, seed=w.seed)).to(dev), 1e-6)
    # the FP6 kernels take 256 x 256 (per-row scales) or 128 x 128 (128-channel
    # groups) tiles, or 32 output columns per workgroup (the decode kernel, 33
    # to 128 or 225 to 256 rows with 128-channel groups): the automatic choice
    # wants at least one workgroup per CU
    fp6_name = w4.outlier_gemm_fp6_kernel_name(M, w.N, w.K, w.n_out, w.group)
    fp6_decode = fp6_name is not None and fp6_name.startswith("gemm_fp6_decode_kernel")
    fp6_tile = 256 if w.group == 0 else 128
    fp6_tiles = -(-w.N // 32) if fp6_decode else -(-M // fp6_tile) * -(-w.N // fp6_tile)
    fp6_fits = fp6_name is not None and (M > 128 or fp6_decode)
    fp6_auto = fp6_fits and fp6_tiles >= 256
    if args.path == "fp6" and not fp6_fits:
        raise SystemExit("the FP6 path takes per-row scales or 128-channel groups (over 32 rows)")
    use_fp6 = args.path == "fp6" or (args.path == "auto" and fp6_auto)
    if use_fp6:
        wf6 = w4.to_fp6(wq)

        def clone_fp6(op):
            return w4.Fp6Operand(*[None if t is None else t.clone() for t in op[:4]], *op[4:])
        plans = [w4.Fp6LayerPlan(Xd.clone(), perm, clone_fp6(wf6), norm=norm) for _ in range(n_sets)]
    else:
        plans = [w4.LayerPlan(Xd.clone(), perm, clone_op(wq), norm=norm) for _ in range(n_sets)]
    # Small decode batches run the layer as one launch (the quantizer, and the
    # RMSNorm with --norm, inside the GEMM's workgroups); every other shape as
    # producer + GEMM (on the FP6 path the producer writes the u6 operand).
    one_launch = not use_fp6 and \
        w4.quant_gemm_kernel_name(M, w.N, w.K, w.n_out, w.group) == "decode_fused_kernel" and \
        (not args.norm or M == 1)

    for i in range(args.warmup):
        p = plans[i % n_sets]
        if one_launch:
            p.fused()
        else:
            p.produce()
            p.gemm()
    torch.cuda.synchronize()

    # How long is a step? One event-timed step after the warmup decides how
    # densely the timed region carries event pairs.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    p = plans[0]
    if one_launch:
        p.fused()
    else:
        p.produce()
        p.gemm()
    e1.record()
    torch.cuda.synchronize()
    every = 1 if e0.elapsed_time(e1) >= LONG_STEP_MS else EVENT_EVERY

    # Timed region: K whole steps. Only the dominant kernel (the GEMM) is
    # bracketed by events, on its launch stream (torch's current stream, which
    # the binding launches on); an event between the producer and the GEMM
    # would itself add a gap to every step.
    K = args.steps
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in range(0, K, every)}
    clock = ClockSampler()
    torch.cuda.synchronize()
    with clock:
        t0 = time.perf_counter()
        for i in range(K):
            p = plans[i % n_sets]
            if not one_launch:
                p.produce()
            e = ev.get(i)
            if e:
                e[0].record()
            if one_launch:
                p.fused()
            else:
                p.gemm()
            if e:
                e[1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / K
    gemm_all = np.array([e[0].elapsed_time(e[1]) for e in ev.values()])
    gemm_ms = float(np.mean(gemm_all))
    p10, p50, p90 = (float(v) * 1e3 for v in np.percentile(gemm_all, [10, 50, 90]))
    # the producer's share, from events around it alone (after the timed region)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(0 if one_launch else min(K, 50))]
    for i, e in enumerate(pev):
        p = plans[i % n_sets]
        e[0].record()
        p.produce()
        e[1].record()
        p.gemm()
    torch.cuda.synchronize()
    prod_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pev])) if pev else None
    ops, gemm_bytes, prod_bytes, one_bytes = work_counts(w, M, args.norm, use_fp6)
    if one_launch:
        gemm_bytes = one_bytes
    value = ops / (ms_step * 1e-3) / 1e12

    mem_bound = ops / gemm_bytes < PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mem_bound:
        ach = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS}
    else:
        ach = ops / (gemm_ms * 1e-3) / 1e12
        # a contraction's peak is that of its own operand type: on the FP6 path
        # the INT4 head runs at the FP6 rate and the INT8 tail at the i8 rate,
        # so the peak is the ops-weighted harmonic combination of the two
        peak = PEAK_INT8_TOPS
        if use_fp6:
            head, tail = 2.0 * M * w.N * w.K_n, 2.0 * M * w.N * w.n_out
            peak = ops / (head / PEAK_FP6_TOPS + tail / PEAK_INT8_TOPS)
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TOP/s", "frac": ach / peak}
    if use_fp6:
        roof["kernel"] = w4.outlier_gemm_fp6_kernel_name(M, w.N, w.K, w.n_out, w.group)
    else:
        roof["kernel"] = (w4.quant_gemm_kernel_name if one_launch else w4.outlier_gemm_kernel_name)(
            M, w.N, w.K, w.n_out, w.group)
    roof["traffic"] = traffic_record(w.name, M, roof["kernel"])

    # the result is checked: the fused call against producer + GEMM (the same
    # bits whether the fused call takes one launch or two); on the FP6 path
    # with the norm, the producer's operand against the nibble norm producer's
    # repacked to u6, and then the fused call without the norm checks the GEMM
    yf = torch.empty_like(plans[0].out)
    chk = plans[0]
    if use_fp6 and norm is not None:
        plans[0].produce()
        ref = w4.to_fp6(w4.rmsnorm_quant_reorder_act(plans[0]._keep[0], norm[0], norm[1], perm, w.n_out, w.group))
        torch.cuda.synchronize()
        got = plans[0].a
        if not (torch.equal(got.u6, ref.u6) and torch.equal(got.s4, ref.s4) and torch.equal(got.s8, ref.s8)
                and (got.q8 is None or torch.equal(got.q8, ref.q8))):
            raise SystemExit("FP6 norm producer and nibble norm producer + repack disagree")
        chk = w4.Fp6LayerPlan(plans[0]._keep[0], perm, plans[0]._keep[2], out=plans[0].out)
    if use_fp6:
        w4.quant_gemm_fp6(chk._keep[0], perm, chk._keep[2], out=yf)
    elif norm is None:
        w4.quant_gemm(plans[0]._keep[0], perm, plans[0]._keep[2], out=yf)
    else:
        w4.rmsnorm_quant_gemm(plans[0]._keep[0], norm[0], norm[1], perm, plans[0]._keep[2], out=yf)
    chk.produce()
    chk.gemm()
    torch.cuda.synchronize()
    if not torch.equal(yf, chk.out):
        raise SystemExit("fused call and producer + GEMM disagree")

    out = {
        "metric": "W4A4+outlier linear TOPS & % INT8-MFMA peak (prefill); GB/s % HBM (decode)",
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 as fp6 e2m3 (exact) + int8 tail" if use_fp6 else "int4 widened to int8 + int8 tail",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "N": w.N, "K": w.K, "n_out": w.n_out,
                   "group": w.group, "buffer_sets": n_sets, "gemm_path": "fp6" if use_fp6 else "i8",
                   "producer": ("rmsnorm_" if args.norm else "") + ("in_gemm" if one_launch else
                                                                     ("fused" if args.norm else "plain"))},
        "roofline": roof,
        "kernels": {
            "producer_us": prod_ms * 1e3 if prod_ms else None,
            "producer_writes_u6": bool(use_fp6),
            "producer_GBps": prod_bytes / (prod_ms * 1e-3) / 1e9 if prod_ms else None,
            "producer_hbm_frac": prod_bytes / (prod_ms * 1e-3) / 1e9 / PEAK_HBM_GBS if prod_ms else None,
            "gemm_us": gemm_ms * 1e3,
            "gemm_us_p10_p50_p90": [p10, p50, p90],
            "gemm_event_pairs": int(gemm_all.size),
            "gemm_TOPS": ops / (gemm_ms * 1e-3) / 1e12,
            "gemm_GBps": gemm_bytes / (gemm_ms * 1e-3) / 1e9,
            "gemm_frac_of_int8_mfma_peak": ops / (gemm_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
        },
        "sclk": sclk_report(clock, profile_record(w.name, M, roof["kernel"]), roof["kernel"]),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, X, W, outliers, args.cpu_budget,
                                           *((norm[0].cpu().numpy(), norm[1]) if norm else ()))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
