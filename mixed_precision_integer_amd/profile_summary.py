"""Summaries of rocprofv3 runs of bench.py for the profiles/ folder.

    python -m mixed_precision_integer_amd.profile_summary DIR WORKLOAD TITLE OUT.md [--m M] [--extra ARGS]
    python -m mixed_precision_integer_amd.profile_summary DIR - TITLE OUT.md --args "BENCH ARGS"

DIR holds the output of five (or six) rocprofv3 runs of bench.py (the
commands are written into the summary):

    DIR/trace   --kernel-trace --stats over the workload
    DIR/fetch   --pmc FETCH_SIZE over the workload
    DIR/write   --pmc WRITE_SIZE over the workload
    DIR/cfetch  --pmc FETCH_SIZE over a plain 512 MiB device copy
    DIR/cwrite  --pmc WRITE_SIZE over the same copy
    DIR/clock   --pmc GRBM_GUI_ACTIVE over the workload (optional: the
                achieved shader clock)

The copy reads and writes exactly 512 MiB, so it gives the scale from the
counters to bytes. The summary is written to profiles/OUT.md, and the GEMM's
HBM bytes per launch are recorded in profiles/gemm_traffic.json under the
workload, with a digest of the GEMM sources: bench.py reports the record as
roofline traffic only while the sources are unchanged.

With ``--args`` (the workload given as ``-``) the runs were made with
``python3 bench.py ARGS`` and the summary covers every kernel of the library
in them (the fused RMSNorm producer, the outlier selection), with no GEMM
traffic record.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# Sources that make up each GEMM kernel (by name prefix): a counter record is
# valid while these are unchanged. Shared headers count for every kernel.
SHARED_SOURCES = ("gemm_common.h", "w4a4_internal.h")
KERNEL_SOURCES = (
    ("gemm_fp6_big_kernel", ("gemm_fp6.hip", "gemm_fp6_common.h", "gemm_fp6_internal.h")),
    ("gemm_fp6_group_kernel", ("gemm_fp6_group.hip", "gemm_fp6_common.h", "gemm_fp6_internal.h")),
    ("gemm_fp6_decode_kernel", ("gemm_fp6_decode.hip", "gemm_fp6_common.h", "gemm_fp6_internal.h")),
    ("gemm_big_kernel", ("gemm_big.hip", "gemm_kernels.hip")),
    ("gemm_group_kernel", ("gemm_group.hip", "gemm_kernels.hip")),
    ("gemm_decode", ("gemm_decode.hip", "gemm_kernels.hip")),
    ("decode_fused_kernel", ("gemm_decode_fused.hip", "gemm_decode.hip", "gemm_kernels.hip")),
    ("gemm_kernel", ("gemm_kernels.hip",)),
)
GEMM_SOURCES = SHARED_SOURCES + tuple(sorted({f for _, fs in KERNEL_SOURCES for f in fs}))
COPY_KIB = 512 * 1024
MAX_SCLK_MHZ = 2400.0 * 1.01                 # the chip's peak engine clock, with rounding room


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed, so that an
    edit of a comment alone leaves the digest (and the counter records) valid.
    String and character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_sources(kernel: str):
    """The source files of a GEMM kernel (its name with or without namespace
    and template arguments), shared headers first."""
    base = kernel.split("(")[0].split("<")[0].split("::")[-1].strip()
    for prefix, files in KERNEL_SOURCES:
        if base.startswith(prefix):
            return SHARED_SOURCES + files
    return GEMM_SOURCES


def gemm_source_digest(kernel: str = "") -> str:
    """First 16 hex digits of the SHA-256 of a GEMM kernel's sources (all GEMM
    sources when no kernel is named; code only, in a fixed order)."""
    h = hashlib.sha256()
    for name in (kernel_sources(kernel) if kernel else GEMM_SOURCES):
        with open(os.path.join(HERE, "csrc", name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_key(workload: str, M: int, kernel: str) -> str:
    """Record key: workload, rows and the GEMM kernel's name (no namespace)."""
    return f"{workload}:M={M}:{kernel.split('(')[0].split('::')[-1]}"


def _csv(folder: str, suffix: str):
    files = glob.glob(os.path.join(folder, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {folder}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _pmc(folder: str, counter: str):
    """Mean counter value per dispatch, by kernel name."""
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for r in _csv(folder, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            tot[r["Kernel_Name"]] += float(r["Counter_Value"])
            disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    return {k: (tot[k] / len(disp[k]), len(disp[k])) for k in tot}


def _clock(folder: str):
    """Per kernel: mean GRBM_GUI_ACTIVE, mean duration (µs) and dispatches of
    a GRBM_GUI_ACTIVE counter run, or {} when there is none."""
    if not os.path.isdir(folder):
        return {}
    tot, dur = collections.defaultdict(float), collections.defaultdict(dict)
    for r in _csv(folder, "counter_collection.csv"):
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            tot[r["Kernel_Name"]] += float(r["Counter_Value"])
            dur[r["Kernel_Name"]][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = {}
    for k, ds in dur.items():
        if "w4a4" in k and ds:
            n = len(ds)
            out[k] = (tot[k] / n, sum(ds.values()) / n, n)
    return out


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def _bench_line(log: str):
    with open(log) as f:
        lines = [l for l in f if l.startswith("{")]
    return json.loads(lines[-1])


def summarize(d: str, workload: str, title: str, out: str, m_arg: str = "", extra: str = "") -> str:
    stats = _csv(os.path.join(d, "trace"), "kernel_stats.csv")
    fetch = _pmc(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _pmc(os.path.join(d, "write"), "WRITE_SIZE")
    cf = _pmc(os.path.join(d, "cfetch"), "FETCH_SIZE")
    cw = _pmc(os.path.join(d, "cwrite"), "WRITE_SIZE")
    ck = next(k for k in cf if "copyBuffer" in k)
    f_scale, w_scale = COPY_KIB / cf[ck][0], COPY_KIB / cw[ck][0]
    bj = _bench_line(os.path.join(d, "trace.log"))
    c = bj["config"]
    gemm_name = bj["roofline"]["kernel"]
    run = f"python3 bench.py --workload {workload}{m_arg}{' ' + extra if extra else ''}"
    L = [f"# {title}\n",
         "Workload: `%s` (M=%d, N=%d, K=%d, n_out=%d, group=%d), seeded synthetic inputs resident in "
         "HBM, buffer sets rotated over more than 512 MB. GEMM kernel for this shape: `%s`.\n"
         % (c["workload"], c["M"], c["N"], c["K"], c["n_out"], c["group"], gemm_name),
         "## Kernel trace (rocprofv3 --kernel-trace --stats)\n",
         "```\ncd /tmp && export TMPDIR=/tmp && cd <repo>\n"
         f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- "
         f"{run} --steps 20 --warmup 5 --no-cpu-baseline\n```\n",
         "| kernel | calls | average µs | min µs | max µs | share of GPU time |",
         "|---|---|---|---|---|---|"]
    for r in stats:
        if "w4a4" in r["Name"]:
            L.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    L.append("\nThe other kernels in the trace (torch set-up copies and fills, the result check) "
             "are not part of a step.\n")
    k = bj["kernels"]
    roof = bj["roofline"]
    prod = ("producer %.2f µs" % k["producer_us"] if k["producer_us"] is not None
            else "producer inside the GEMM kernel (one launch)")
    L.append("bench.py line printed in the same run (HIP events on the launch stream around every eighth "
             "GEMM launch of the timed region): %s, GEMM %.2f µs, step %.2f µs, value %.1f %s; "
             "roofline: %.1f of %.0f %s (%.1f%%, %s-bound).\n"
             % (prod, k["gemm_us"], bj["ms_per_step"] * 1e3, bj["value"], bj["unit"],
                roof["achieved"], roof["peak"], roof["unit"], 100 * roof["frac"], roof["bound"]))
    L.append("## HBM traffic (rocprofv3 --pmc, one counter per run)\n")
    cmds = [("FETCH_SIZE", "fetch", f"{run} --steps 5 --warmup 2 --no-cpu-baseline"),
            ("WRITE_SIZE", "write", f"{run} --steps 5 --warmup 2 --no-cpu-baseline"),
            ("FETCH_SIZE", "cfetch", "python3 bench.py --copy-probe-mib 512 --steps 5 --warmup 2"),
            ("WRITE_SIZE", "cwrite", "python3 bench.py --copy-probe-mib 512 --steps 5 --warmup 2")]
    L.append("```\n" + "\n".join(
        f"timeout -s KILL 120 rocprofv3 --pmc {cn} --output-format csv -d {d}/{o} -o p -- {cmd}"
        for cn, o, cmd in cmds) + "\n```\n")
    L.append(f"Calibration: the plain 512 MiB device copy (`{_short(ck)}`, {cf[ck][1]} dispatches) reads "
             f"{cf[ck][0]:.0f} KiB (FETCH_SIZE) and writes {cw[ck][0]:.0f} KiB (WRITE_SIZE) per dispatch "
             f"for {COPY_KIB} KiB moved each way, so bytes = FETCH_SIZE x {f_scale:.3f} KiB and "
             f"WRITE_SIZE x {w_scale:.3f} KiB.\n")
    L.append("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | "
             "total MB per launch |")
    L.append("|---|---|---|---|---|---|---|")
    traffic = {}
    for kn, (fk, n) in fetch.items():
        if "w4a4" not in kn:
            continue
        wk = write.get(kn, (0.0, 0))[0]
        rb, wb = fk * f_scale * 1024, wk * w_scale * 1024
        traffic[_short(kn)] = rb + wb
        L.append(f"| `{_short(kn)}` | {n} | {fk:.0f} | {wk:.0f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} | "
                 f"{(rb + wb) / 1e6:.2f} |")
    clock = _clock(os.path.join(d, "clock"))
    if clock:
        L.append("\n## Achieved shader clock (rocprofv3 --pmc GRBM_GUI_ACTIVE)\n")
        L.append("```\ntimeout -s KILL 120 rocprofv3 --pmc GRBM_GUI_ACTIVE --output-format csv -d "
                 f"{d}/clock -o p -- {run} --steps 5 --warmup 2 --no-cpu-baseline\n```\n")
        L.append("GRBM_GUI_ACTIVE counts the cycles the graphics engine is busy, summed over the eight XCDs; "
                 "divided by 8 and by the dispatch's duration (the counter run's own timestamps) it gives the "
                 "average shader clock while the kernel ran.\n")
        L.append("For dispatches of a few tens of µs the counter also takes in cycles around the dispatch, so "
                 "the quotient can exceed the 2400 MHz the chip runs at; such values are marked and not "
                 "recorded.\n")
        L.append("| kernel | dispatches | GRBM_GUI_ACTIVE | average duration µs | clock MHz |")
        L.append("|---|---|---|---|---|")
        for kn, (g, dur, n) in clock.items():
            mhz = g / 8 / dur
            note = "" if mhz <= MAX_SCLK_MHZ else " (not a clock: above the chip's 2400)"
            L.append(f"| `{_short(kn)}` | {n} | {g:.0f} | {dur:.2f} | {mhz:.0f}{note} |")
    text = "\n".join(L) + "\n"
    with open(os.path.join(ROOT, "profiles", out), "w") as f:
        f.write(text)
    base = gemm_name.split("<")[0].split(" ")[0]
    gk = [kk for kk in traffic if kk.split("::")[-1].split("<")[0] == base]
    if gk:
        p = os.path.join(ROOT, "profiles", "gemm_traffic.json")
        rec = json.load(open(p)) if os.path.exists(p) else {}
        rec[traffic_key(c["workload"], c["M"], gk[0])] = {
            "gemm_sources_sha256_16": gemm_source_digest(gk[0]), "kernel": gk[0],
            "hbm_bytes_per_launch": traffic[gk[0]], "fetch_scale_kib": f_scale,
            "write_scale_kib": w_scale, "profile": out}
        ck_k = [kk for kk in clock if _short(kk) == gk[0]]
        if ck_k:
            g, dur, _ = clock[ck_k[0]]
            if g / 8 / dur <= MAX_SCLK_MHZ:
                rec[traffic_key(c["workload"], c["M"], gk[0])]["sclk_mhz"] = g / 8 / dur
        with open(p, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
    return text


def summarize_kernels(d: str, bench_args: str, title: str, out: str) -> str:
    """Kernel trace and HBM traffic of every library kernel in a bench.py run
    made with `bench_args` (no GEMM traffic record)."""
    stats = _csv(os.path.join(d, "trace"), "kernel_stats.csv")
    fetch = _pmc(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _pmc(os.path.join(d, "write"), "WRITE_SIZE")
    cf = _pmc(os.path.join(d, "cfetch"), "FETCH_SIZE")
    cw = _pmc(os.path.join(d, "cwrite"), "WRITE_SIZE")
    ck = next(k for k in cf if "copyBuffer" in k)
    f_scale, w_scale = COPY_KIB / cf[ck][0], COPY_KIB / cw[ck][0]
    bj = _bench_line(os.path.join(d, "trace.log"))
    run = f"python3 bench.py {bench_args}"
    L = [f"# {title}\n",
         f"bench.py configuration: `{json.dumps(bj['config'])}`; seeded synthetic inputs resident in HBM, "
         "buffer sets rotated over more than 512 MB.\n",
         "## Kernel trace (rocprofv3 --kernel-trace --stats)\n",
         "```\ncd /tmp && export TMPDIR=/tmp && cd <repo>\n"
         f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- "
         f"{run} --steps 20 --warmup 5 --no-cpu-baseline\n```\n",
         "| kernel | calls | average µs | min µs | max µs | share of GPU time |",
         "|---|---|---|---|---|---|"]
    avg = {}
    for r in stats:
        if "w4a4" in r["Name"]:
            avg[_short(r["Name"])] = float(r["AverageNs"]) / 1e3
            L.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    L.append("\nThe other kernels in the trace (torch set-up copies and fills) are not part of a step.\n")
    roof = bj["roofline"]
    line = (f"bench.py line printed in the same run: value {bj['value']:.1f} {bj['unit']}, "
            f"{bj['ms_per_step'] * 1e3:.2f} µs per step; roofline {roof['achieved']:.1f} of "
            f"{roof['peak']:.0f} {roof['unit']} ({100 * roof['frac']:.1f}%, {roof['bound']}-bound, "
            f"{roof['kernel']})")
    if "kernels" in bj:
        # numbers only (the line also carries flags and percentile lists)
        line += "; " + ", ".join(f"{key} {val:.2f}" for key, val in bj["kernels"].items()
                                 if isinstance(val, (int, float)) and not isinstance(val, bool))
    L.append(line + ".\n")
    L.append("## HBM traffic (rocprofv3 --pmc, one counter per run)\n")
    cmds = [("FETCH_SIZE", "fetch", f"{run} --steps 5 --warmup 2 --no-cpu-baseline"),
            ("WRITE_SIZE", "write", f"{run} --steps 5 --warmup 2 --no-cpu-baseline"),
            ("FETCH_SIZE", "cfetch", "python3 bench.py --copy-probe-mib 512 --steps 5 --warmup 2"),
            ("WRITE_SIZE", "cwrite", "python3 bench.py --copy-probe-mib 512 --steps 5 --warmup 2")]
    L.append("```\n" + "\n".join(
        f"timeout -s KILL 120 rocprofv3 --pmc {cn} --output-format csv -d {d}/{o} -o p -- {cmd}"
        for cn, o, cmd in cmds) + "\n```\n")
    L.append(f"Calibration: the plain 512 MiB device copy (`{_short(ck)}`) reads {cf[ck][0]:.0f} KiB "
             f"(FETCH_SIZE) and writes {cw[ck][0]:.0f} KiB (WRITE_SIZE) per dispatch for {COPY_KIB} KiB "
             f"moved each way: bytes = FETCH_SIZE x {f_scale:.3f} KiB and WRITE_SIZE x {w_scale:.3f} KiB.\n")
    L.append("| kernel | dispatches | HBM read MB | HBM write MB | total MB per launch | GB/s at the trace's "
             "average duration |")
    L.append("|---|---|---|---|---|---|")
    for kn, (fk, n) in fetch.items():
        if "w4a4" not in kn:
            continue
        wk = write.get(kn, (0.0, 0))[0]
        rb, wb = fk * f_scale * 1024, wk * w_scale * 1024
        t = avg.get(_short(kn))
        rate = f"{(rb + wb) / (t * 1e-6) / 1e9:.0f}" if t else "-"
        L.append(f"| `{_short(kn)}` | {n} | {rb / 1e6:.2f} | {wb / 1e6:.2f} | {(rb + wb) / 1e6:.2f} | {rate} |")
    text = "\n".join(L) + "\n"
    with open(os.path.join(ROOT, "profiles", out), "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("workload")
    ap.add_argument("title")
    ap.add_argument("out")
    ap.add_argument("--m", default=None, help="the --m argument the runs were made with")
    ap.add_argument("--args", default=None, help="bench.py arguments of a kernel-summary run")
    ap.add_argument("--extra", default="", help="further bench.py arguments of the runs (e.g. --path i8)")
    a = ap.parse_args()
    if a.args is not None:
        print(summarize_kernels(os.path.relpath(a.dir, ROOT) if os.path.isabs(a.dir) else a.dir, a.args,
                                a.title, a.out))
        return
    print(summarize(os.path.relpath(a.dir, ROOT) if os.path.isabs(a.dir) else a.dir, a.workload, a.title,
                    a.out, f" --m {a.m}" if a.m else "", a.extra))


if __name__ == "__main__":
    main()
