"""Summaries of rocprofv3 runs of ``bench.py`` for the ``profiles/`` folder.

Two kinds of run are summarised (the commands are recorded in each summary):

* ``stats``: ``rocprofv3 --kernel-trace --stats -f csv ... -- python3 bench.py``.
  The summary lists every kernel's call count and mean duration, and puts the
  mean duration rocprofv3 measured for the roofline kernel next to the mean
  the bench measured with HIP events in the same run.
* ``pmc``: two ``rocprofv3 --pmc`` runs of the bench, one with ``FETCH_SIZE``
  and one with ``WRITE_SIZE``.  Each counter is scaled by what it reads for the
  bench's calibration copy (``stream_copy_kernel``, a plain copy of a known
  number of bytes), and the scaled HBM bytes per launch of the roofline kernel
  are written to a JSON file that ``bench.py`` reports as ``roofline.traffic``
  while the kernel sources still hash to the recorded value.
* ``mfma``: one ``rocprofv3 --pmc`` run of the bench with the INT8 MFMA counters
  ``SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_I8 SQ_VALU_MFMA_BUSY_CYCLES
  GRBM_GUI_ACTIVE``.  Per linear kernel: MFMA instructions and executed INT8
  ops per dispatch (MOPS x 512), ops per instruction (32768 for the 16x16x64
  INT8 MFMA: a check of the scaling), the MFMA busy share of the SIMDs' cycles
  while the GPU was active, and the executed TOP/s at the bench's launch time.

    python -m w8a8_quantized_speculative_amd.profiling stats STATS_CSV BENCH_JSON OUT_MD --command CMD [--trace TRACE_CSV]
    python -m w8a8_quantized_speculative_amd.profiling pmc FETCH_CSV WRITE_CSV BENCH_JSON OUT_JSON OUT_MD \\
        --command-fetch CMD --command-write CMD
    python -m w8a8_quantized_speculative_amd.profiling mfma PMC_CSV BENCH_JSON OUT_MD --command CMD
"""
from __future__ import annotations

import argparse
import csv
import shlex
import sys
import hashlib
import json
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
# the file that defines each kernel family; every family also depends on the
# shared device headers
_FAMILY_SOURCES = (
    ("w8a8_linear_fused_kernel", "fused.hip"),
    ("w4a8_linear_fused_kernel", "fused.hip"),
    ("w8a8_linear_wide_kernel", "wide.hip"),
    ("w4a8_linear_wide_kernel", "wide.hip"),
    ("w8a8_linear_wide_split_kernel", "wide.hip"),
    ("w4a8_linear_wide_split_kernel", "wide.hip"),
    ("w8a8_chain_kernel", "chain.hip"),
    ("accept_", "accept.hip"),
)
_SHARED_HEADERS = ("quasar_device.hpp", "quasar_internal.hpp", "quasar_sync.hpp")
COPY_KERNEL = "stream_copy_kernel"


def code_only(text: str) -> str:
    """C++ source text without its comments, whitespace runs collapsed to one
    space (string and character literals kept as written)."""
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


def kernel_source_hash(kernel: str = "w8a8_linear_fused_kernel") -> str:
    """Hash of the code a kernel is built from (its family's file and the
    shared device headers, comments and layout left out): a recorded counter
    reading stays valid while this hash is unchanged."""
    files = [f for prefix, f in _FAMILY_SOURCES if kernel.startswith(prefix)][:1]
    h = hashlib.sha256()
    for name in files + list(_SHARED_HEADERS):
        with open(os.path.join(PKG, "csrc", name), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    """'void ns::(anonymous namespace)::foo<6, 2>(args)' -> 'foo<6, 2>': drop the
    argument list and the qualifiers at template depth 0."""
    depth, cut, last_sep = 0, len(name), 0
    i = 0
    while i < len(name):
        ch = name[i]
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif depth == 0 and name.startswith("(anonymous namespace)", i):
            i += len("(anonymous namespace)")
            continue
        elif depth == 0 and ch == "(":
            cut = i
            break
        elif depth == 0 and name.startswith("::", i):
            last_sep = i + 2
            i += 2
            continue
        i += 1
    head = name[last_sep:cut]
    if head.startswith("void "):
        head = head[5:]
    return head.strip()


def _cell(name: str, width: int = 72) -> str:
    return name if len(name) <= width else name[:width - 3] + "..."


def _bench_line(path: str) -> dict:
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def _self_command() -> str:
    return "python -m w8a8_quantized_speculative_amd.profiling " + " ".join(
        shlex.quote(a) for a in sys.argv[1:])


def _trace_means(trace_csv: str, names) -> dict:
    """Per kernel (short name): the mean duration in ns of its dispatches in the
    launch configuration (grid size, LDS bytes) it was dispatched with most
    often, with the count of those dispatches and of all its dispatches.  The
    step's shapes of a kernel share one configuration, while other sections of
    the bench (the single 1024 x 1024 linear, the tensor-parallel shards) launch
    the same kernel with other grids or LDS sizes."""
    want = set(names)
    groups = defaultdict(lambda: defaultdict(list))
    with open(trace_csv) as f:
        rd = csv.DictReader(f)
        cols = rd.fieldnames or []
        gcol = next((c for c in cols if c.startswith("Grid_Size") and c.endswith("X")),
                    next((c for c in cols if c.startswith("Grid_Size")), None))
        lcol = next((c for c in cols if c in ("LDS_Block_Size", "Group_Segment_Size",
                                               "LDS_Size")), None)
        for r in rd:
            name = _short(r["Kernel_Name"])
            if name not in want:
                continue
            key = (r.get(gcol, ""), r.get(lcol, ""))
            groups[name][key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for name, g in groups.items():
        key, durs = max(g.items(), key=lambda kv: len(kv[1]))
        out[name] = {"mean_ns": sum(durs) / len(durs), "dispatches": len(durs),
                     "all_dispatches": sum(len(v) for v in g.values()),
                     "grid": key[0], "lds": key[1]}
    return out


def summarize_stats(stats_csv: str, bench_json: str, out_md: str, command: str,
                    trace_csv: str | None = None) -> dict:
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((_short(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(key=lambda r: -r[2])
    bench = _bench_line(bench_json)
    roof = bench["roofline"]
    kname = roof["kernel"]
    prof = [r for r in rows if r[0] == kname]
    prof_avg_us = prof[0][3] / 1e3 if prof else None
    others_names = [bench[k]["roofline"]["kernel"] for k in bench if k.startswith("window_m")]
    if "w4a8_variant" in bench and bench["w4a8_variant"].get("kernels"):
        others_names.append(bench["w4a8_variant"]["kernels"][0]["kernel"])
    tm = _trace_means(trace_csv, [kname] + others_names) if trace_csv else {}
    out = ["# rocprofv3 kernel statistics: " + bench["config"]["workload"], "",
           "Profiled command (paths relative to the repository root of the GPU run):", "",
           "```", command, "```", "", "Summary written by:", "", "```", _self_command(), "```", "",
           f"Bench line of the same run: value {bench['value']} {bench['unit']}, "
           f"{bench['ms_per_step']} ms per step, roofline kernel `{kname}`.", "",
           "| kernel | calls | total ms | mean us | min us | max us |",
           "|---|---:|---:|---:|---:|---:|"]
    for name, calls, tot, avg, mn, mx in rows[:20]:
        out.append(f"| `{_cell(name)}` | {calls} | {tot / 1e6:.3f} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                   f"{mx / 1e3:.2f} |")
    t = tm.get(kname)
    out += ["", "Roofline kernel, mean duration per launch:", ""]
    if t:
        lds = f", {t['lds']} B of LDS" if t["lds"] not in ("", "0") else ""
        out.append(f"- rocprofv3, the {t['dispatches']} of its {t['all_dispatches']} dispatches with the "
                   f"launch grid of the step's shapes ({t['grid']} threads{lds}; the other dispatches "
                   f"are smaller grids: the single 1024 x 1024 linear and tensor-parallel shards): "
                   f"{t['mean_ns'] / 1e3:.2f} us")
    out += [
            f"- rocprofv3 (all launches in the run, graph replays and eager calls): "
            f"{prof_avg_us:.2f} us" if prof_avg_us is not None else "- rocprofv3: kernel not found",
            f"- bench.py, HIP events around back-to-back batches of its launches, same run: "
            f"{roof['launch_avg_us']} us",
            f"- algorithmic bytes per launch: {roof['algorithmic_bytes_per_launch']} "
            f"-> {roof['achieved']} GB/s by the events, "
            + (f"{roof['algorithmic_bytes_per_launch'] / ((t['mean_ns'] if t else prof_avg_us * 1e3)):.1f} "
               f"GB/s by rocprofv3" if prof_avg_us else "n/a"),
            ""]
    others = []
    for key in sorted(k for k in bench if k.startswith("window_m")):
        r = bench[key]["roofline"]
        others.append((f"{key} roofline kernel", r["kernel"], r["launch_avg_us"],
                       r["algorithmic_bytes_per_launch"]))
    if "w4a8_variant" in bench and bench["w4a8_variant"].get("kernels"):
        k0 = bench["w4a8_variant"]["kernels"][0]
        others.append(("w4a8_variant dominant kernel", k0["kernel"], k0["launch_avg_us"],
                       k0["algorithmic_bytes_per_launch"]))
    if others:
        out += ["Other measured kernels of the same run (mean per launch; the bench's figure is "
                "mix-weighted over the shapes of its step, as are rocprofv3's launches):", "",
                "| section | kernel | rocprofv3 mean us | bench.py events us | GB/s (rocprofv3) |",
                "|---|---|---:|---:|---:|"]
        by_name = {r[0]: r for r in rows}
        for what, name, ev_us, alg in others:
            pr = by_name.get(name)
            p_us = pr[3] / 1e3 if pr else None
            if name in tm:
                p_us = tm[name]["mean_ns"] / 1e3
            out.append(f"| {what} | `{_cell(name)}` | {p_us:.2f} | {ev_us} | "
                       f"{alg / (p_us * 1e3):.1f} |" if p_us else
                       f"| {what} | `{_cell(name)}` | - | {ev_us} | - |")
        out.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    return {"rocprof_avg_us": prof_avg_us, "events_avg_us": roof["launch_avg_us"],
            "rocprof_step_config_avg_us": (t["mean_ns"] / 1e3) if t else None}


def _counter_means(path: str, counter: str) -> dict:
    """Mean counter value per dispatch, by short kernel name."""
    acc = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name", "").strip() != counter:
                continue
            acc[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_pmc(fetch_csv: str, write_csv: str, bench_json: str, out_json: str, out_md: str,
                  command_fetch: str, command_write: str) -> dict:
    """HBM traffic per launch of every linear kernel of the bench's step (and of
    the 4-bit variant's, when it ran), scaled by the calibration copy."""
    bench = _bench_line(bench_json)
    copy_bytes = bench["copy_calibration"]["bytes"]
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    cf, cw = fetch[COPY_KERNEL][0], write[COPY_KERNEL][0]
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw  # bytes per counter unit
    step_kernels = list(bench.get("kernels", []))
    step_kernels += list(bench.get("w4a8_variant", {}).get("kernels", []))
    kernels = {}
    for k in step_kernels:
        name = k["kernel"]
        if name not in fetch or name not in write:
            continue
        kf, nf = fetch[name]
        kw, nw = write[name]
        traffic = kf * f_scale + kw * w_scale
        alg = k["algorithmic_bytes_per_launch"]
        kernels[name] = {
            "kernel_source_hash": kernel_source_hash(name),
            "traffic_bytes_per_launch": round(traffic),
            "fetch_bytes_per_launch": round(kf * f_scale),
            "write_bytes_per_launch": round(kw * w_scale),
            "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round(traffic / alg, 4),
            "dispatches_averaged": {"FETCH_SIZE": nf, "WRITE_SIZE": nw},
        }
    # cross-check of the FETCH scale on a second kernel of known bytes: the
    # streaming read kernel (the 1 GiB calibration read and the step's
    # read-only twin, bench.py's read_calibration and read_twin)
    rc, rt = bench.get("read_calibration", {}), bench.get("read_twin", {})
    xcheck = None
    if "stream_read_kernel" in fetch and rc.get("dispatches") and rt.get("passes"):
        n_disp = rc["dispatches"] + rt["passes"] * rt["launches_per_pass"]
        expect = (rc["dispatches"] * rc["bytes"] + rt["passes"] * rt["bytes"]) / n_disp
        got = fetch["stream_read_kernel"][0] * f_scale
        xcheck = {"kernel": "stream_read_kernel", "dispatches": fetch["stream_read_kernel"][1],
                  "expected_dispatches": n_disp, "read_bytes_per_dispatch": round(expect),
                  "scaled_fetch_per_dispatch": round(got),
                  "ratio": round(got / expect, 4)}
    res = {
        "workload": bench["config"]["workload"],
        "M": bench["config"]["M"],
        "roofline_kernel": bench["roofline"]["kernel"],
        "kernels": kernels,
        "calibration": {"kernel": COPY_KERNEL, "bytes": copy_bytes,
                        "FETCH_SIZE": cf, "WRITE_SIZE": cw,
                        "bytes_per_unit_fetch": round(f_scale, 4),
                        "bytes_per_unit_write": round(w_scale, 4)},
        "fetch_cross_check": xcheck,
        "commands": [command_fetch, command_write],
        "note": "FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by its reading for a "
                "plain copy of a known size; mean over every launch of the kernel in the run "
                "(the step's mix of shapes)",
    }
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    out = ["# HBM traffic (rocprofv3 PMC): " + bench["config"]["workload"], "",
           "Profiled commands (paths relative to the repository root of the GPU run):", "",
           "```", command_fetch, command_write, "```", "", "Summary written by:", "", "```",
           _self_command(), "```", "",
           f"Calibration: `{COPY_KERNEL}` copies {copy_bytes} bytes; it reads FETCH_SIZE {cf:.1f} "
           f"and WRITE_SIZE {cw:.1f}, i.e. {f_scale:.2f} and {w_scale:.2f} bytes per counter unit.",
           "",
           (f"Cross-check of the FETCH scale on `stream_read_kernel` (the 1 GiB calibration read "
            f"and the step's read-only twin, {xcheck['dispatches']} dispatches, "
            f"{xcheck['expected_dispatches']} expected): {xcheck['scaled_fetch_per_dispatch']} B "
            f"fetched per dispatch against {xcheck['read_bytes_per_dispatch']} B read, ratio "
            f"{xcheck['ratio']}." if xcheck else "No second calibration kernel in this run."),
           "",
           "Linear kernels of the step (mean per launch over the step's mix of shapes):", "",
           "| kernel | dispatches | FETCH bytes/launch | WRITE bytes/launch | traffic | algorithmic | ratio |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for name, r in kernels.items():
        out.append(f"| `{name}` | {r['dispatches_averaged']['FETCH_SIZE']} | "
                   f"{r['fetch_bytes_per_launch']} | {r['write_bytes_per_launch']} | "
                   f"{r['traffic_bytes_per_launch']} | {r['algorithmic_bytes_per_launch']} | "
                   f"{r['traffic_over_algorithmic']:.4f} |")
    out += ["", "Every kernel of the run (scaled the same way, bytes per dispatch):", "",
            "| kernel | dispatches | FETCH | WRITE |", "|---|---:|---:|---:|"]
    for name in sorted(set(fetch) & set(write), key=lambda n: -fetch[n][0] * fetch[n][1]):
        out.append(f"| `{_cell(name)}` | {fetch[name][1]} | {fetch[name][0] * f_scale:.0f} | "
                   f"{write[name][0] * w_scale:.0f} |")
    out.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    return res


SIMDS = 1024        # MI355X: 256 compute units x 4 SIMDs
PEAK_INT8_TOPS = 5000.0


def kernel_launch_times(bench: dict) -> dict:
    """kernel name -> its entry (launch_avg_us, algorithmic ops...) from every
    section of a bench line that lists kernels: the step's, each window's and
    each 4-bit variant's."""
    out = {}

    def walk(d):
        if isinstance(d, dict):
            for k in d.get("kernels", []) if isinstance(d.get("kernels"), list) else []:
                if isinstance(k, dict) and "kernel" in k:
                    out.setdefault(k["kernel"], k)
            for v in d.values():
                if isinstance(v, dict):
                    walk(v)
    walk(bench)
    return out


def summarize_mfma(pmc_csv: str, bench_json: str, out_md: str, command: str,
                   timing_json: str = None) -> dict:
    """MFMA counters per kernel.  Launch times come from `timing_json` (a bench
    line of a run without counters) when given: the counter runs serialize the
    dispatches and time each launch several times longer."""
    bench = _bench_line(bench_json)
    mops = _counter_means(pmc_csv, "SQ_INSTS_VALU_MFMA_MOPS_I8")
    insts = _counter_means(pmc_csv, "SQ_INSTS_VALU_MFMA_I8")
    busy = _counter_means(pmc_csv, "SQ_VALU_MFMA_BUSY_CYCLES")
    active = _counter_means(pmc_csv, "GRBM_GUI_ACTIVE")
    launch_us = kernel_launch_times(_bench_line(timing_json) if timing_json else bench)
    rows, res = [], {}
    for name in sorted(mops, key=lambda n: -mops[n][0] * mops[n][1]):
        if not (name.startswith("w8a8_linear") or name.startswith("w4a8_linear")):
            continue
        ops = mops[name][0] * 512
        ni = insts.get(name, (0, 0))[0]
        b = busy.get(name, (0, 0))[0]
        a = active.get(name, (0, 0))[0]
        util = b / (a * SIMDS) if a else 0.0
        k = launch_us.get(name)
        tops = ops / (k["launch_avg_us"] * 1e-6) / 1e12 if k else None
        alg = k.get("algorithmic_int8_ops_per_launch") if k else None
        res[name] = {"dispatches": mops[name][1], "mfma_insts_per_dispatch": round(ni),
                     "executed_int8_ops_per_dispatch": round(ops),
                     "ops_per_inst": round(ops / ni, 1) if ni else None,
                     "mfma_busy_frac_counter_run": round(util, 4),
                     "executed_tops": round(tops, 2) if tops else None,
                     "executed_frac_of_peak": round(tops / PEAK_INT8_TOPS, 4) if tops else None,
                     "algorithmic_int8_ops_per_launch_in_step": alg}
        rows.append(f"| `{_cell(name)}` | {mops[name][1]} | {ni:.0f} | {ops:.3e} | "
                    f"{(ops / ni) if ni else 0:.0f} | {100 * util:.2f}% | "
                    f"{(f'{tops:.1f}') if tops else '-'} | "
                    f"{(f'{100 * tops / PEAK_INT8_TOPS:.1f}%') if tops else '-'} | "
                    f"{(f'{alg:.3e}') if alg else '-'} |")
    out = ["# INT8 MFMA use (rocprofv3 PMC): " + bench["config"]["workload"], "",
           "Profiled command (paths relative to the repository root of the GPU run):", "",
           "```", command, "```", "", "Summary written by:", "", "```", _self_command(), "```", "",
           "Per dispatch, mean over every launch of the kernel in the run (the bench's mix of "
           "shapes).  Executed ops = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512; they include the MFMA "
           "work on padding (token columns past M, channels past N), so they exceed the "
           "algorithmic 2*M*N*K.  TOP/s = executed ops / the kernel's mean launch time in "
           + ("a bench run without counters" if timing_json else "the same run")
           + f", and its share of the dense INT8 peak ({PEAK_INT8_TOPS:.0f} TOP/s) is the "
           "matrix units' use.  MFMA busy (counter run) = SQ_VALU_MFMA_BUSY_CYCLES / "
           f"(GRBM_GUI_ACTIVE x {SIMDS} SIMDs) during the counter run, which serializes the "
           "dispatches and stretches each several times, so it understates the use by that "
           "factor.", "",
           "| kernel | dispatches | MFMA insts | executed INT8 ops | ops/inst | MFMA busy "
           "(counter run) | executed TOP/s | share of INT8 peak | algorithmic ops/launch "
           "(step mix) |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"] + rows + [""]
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("stats_csv")
    a.add_argument("bench_json")
    a.add_argument("out_md")
    a.add_argument("--command", required=True)
    a.add_argument("--trace", default=None, help="kernel_trace.csv of the same run")
    b = sub.add_parser("pmc")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("bench_json")
    b.add_argument("out_json")
    b.add_argument("out_md")
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    c = sub.add_parser("mfma")
    c.add_argument("pmc_csv")
    c.add_argument("bench_json")
    c.add_argument("out_md")
    c.add_argument("--command", required=True)
    c.add_argument("--timing", default=None,
                   help="bench line of a run without counters, for the launch times")
    args = ap.parse_args()
    if args.cmd == "mfma":
        print(json.dumps(summarize_mfma(args.pmc_csv, args.bench_json, args.out_md,
                                        args.command, args.timing)))
    elif args.cmd == "stats":
        print(json.dumps(summarize_stats(args.stats_csv, args.bench_json, args.out_md,
                                         args.command, args.trace)))
    else:
        print(json.dumps(summarize_pmc(args.fetch_csv, args.write_csv, args.bench_json,
                                       args.out_json, args.out_md, args.command_fetch,
                                       args.command_write)))


if __name__ == "__main__":
    main()
